// api.hip -- the C ABI declared in include/nsa_sel.h: descriptor checks,
// workspace planning and the launch sequences.  Host code only.
#include "../../include/nsa_sel.h"
#include "internal.h"

#include <stdio.h>

#include <algorithm>
#include <mutex>

#ifndef NSA_IDX_MIN_TILE
#define NSA_IDX_MIN_TILE 128
#endif

namespace nsa {
hipError_t launch_index(const Params& p, int32_t* offsets, int32_t* entries, hipStream_t st);
hipError_t launch_index_prebuilt(const Params& p, const int32_t* offsets_in, const int32_t* entries_in, int cap,
                                 hipStream_t st);
hipError_t launch_main(const Params& p, int kind, hipStream_t st);
hipError_t launch_merge(const Params& p, int kind, hipStream_t st);
hipError_t launch_dense(const Params& p, int kind, hipStream_t st);
int main_grid_size(int D, int bs, int kind);
hipError_t launch_bwd_delta(const Params& p, int kind, hipStream_t st);
hipError_t launch_bwd_main(const Params& p, int kind, hipStream_t st);
hipError_t launch_bwd_dq_merge(const Params& p, int kind, hipStream_t st);
int bwd_grid_size(int D, int bs, int kind);
hipError_t launch_prep(const Params& p, hipStream_t st);
hipError_t launch_window(const Params& p, int kind, hipStream_t st);
hipError_t launch_window_orphans(const Params& p, int kind, hipStream_t st);
hipError_t launch_sel_prep(const Params& p, hipStream_t st);
hipError_t launch_compress(const Params& p, int kind, hipStream_t st);
hipError_t launch_select(const Params& p, int kind, int32_t* order, hipStream_t st);
int64_t select_max_tiles(int64_t T, int B, int G);
hipError_t launch_sel_orphans(const Params& p, hipStream_t st);
bool select_supported(int D, int G, int bs, int ks, int stride);
int select_cap(int64_t T, int B);
int select_tokens(int G, int topk, int init, int local);
}  // namespace nsa

namespace {

using nsa::div_up;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Plan {
    int64_t T;
    int B, Hq, Hkv, G, D, bs, topk;
    int nbc, ntiles, tile_tokens, item_rows;
    int64_t max_items;
    size_t elt;  // bytes per q/k/v/out element
    // workspace offsets
    size_t o_status, o_cus, o_blkoff, o_tilecnt, o_counts, o_item_start, o_offsets, o_entries;
    size_t o_item_bucket, o_slot_pos, o_dense_cnt, o_dense_ids, o_dense_o, o_dense_lse;
    size_t o_part_lse, o_part_o;
    size_t index_bytes;  // end of what the inversion alone needs
    size_t fwd_bytes;
    // backward: index part as above (offsets, entries), then
    size_t o_bslot_pos, o_delta, o_dkv_part, o_dq_part;
    size_t bwd_bytes;
};

int elem_kind(int dtype)
{
    return dtype == NSA_SEL_DTYPE_BF16 ? nsa::kElemBF16 : dtype == NSA_SEL_DTYPE_F16 ? nsa::kElemF16 : nsa::kElemF32;
}

int check_desc(const nsa_sel_desc* d)
{
    if (!d) return NSA_SEL_ERR_INVALID_ARG;
    if (d->struct_size != sizeof(nsa_sel_desc)) return NSA_SEL_ERR_INVALID_ARG;
    if (d->num_seqs < 1 || d->total_tokens < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
        d->head_dim < 1 || d->block_size < 1 || d->topk < 1)
        return NSA_SEL_ERR_INVALID_ARG;
    if (d->num_q_heads % d->num_kv_heads != 0) return NSA_SEL_ERR_INVALID_ARG;
    if (!(d->scale == d->scale)) return NSA_SEL_ERR_INVALID_ARG;  // NaN
    if (d->flags & ~NSA_SEL_FLAG_DENSE_SPLIT) return NSA_SEL_ERR_INVALID_ARG;
    if (d->dtype != NSA_SEL_DTYPE_BF16 && d->dtype != NSA_SEL_DTYPE_F16 && d->dtype != NSA_SEL_DTYPE_F32)
        return NSA_SEL_ERR_UNSUPPORTED;
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return NSA_SEL_ERR_UNSUPPORTED;
    if (d->block_size != 32 && d->block_size != 64 && d->block_size != 128) return NSA_SEL_ERR_UNSUPPORTED;
    // d = 256: 16-bit inputs (the backward also blocks of at most 64 keys)
    if (d->head_dim == 256 && d->dtype == NSA_SEL_DTYPE_F32) return NSA_SEL_ERR_UNSUPPORTED;
    if (d->topk > 64) return NSA_SEL_ERR_UNSUPPORTED;
    const int G = d->num_q_heads / d->num_kv_heads;
    if (G > 64) return NSA_SEL_ERR_UNSUPPORTED;
    const int64_t T = d->total_tokens;
    if (T > INT32_MAX / 2) return NSA_SEL_ERR_UNSUPPORTED;
    if (T * d->num_q_heads * (int64_t)d->topk >= ((int64_t)1 << 31)) return NSA_SEL_ERR_UNSUPPORTED;
    const int64_t nbc = T / d->block_size + d->num_seqs;
    if (nbc * d->num_kv_heads >= ((int64_t)1 << 31)) return NSA_SEL_ERR_UNSUPPORTED;
    return NSA_SEL_OK;
}

int make_plan(const nsa_sel_desc* d, Plan* pl)
{
    int rc = check_desc(d);
    if (rc != NSA_SEL_OK) return rc;
    Plan& P = *pl;
    P.T = d->total_tokens;
    P.B = d->num_seqs;
    P.Hq = d->num_q_heads;
    P.Hkv = d->num_kv_heads;
    P.G = P.Hq / P.Hkv;
    P.D = d->head_dim;
    P.bs = d->block_size;
    P.topk = d->topk;
    P.nbc = (int)(P.T / P.bs + P.B);
    // token tiles of the inversion: the smallest power of two from 64 tokens
    // that keeps the (kv head, tile, bucket) table within 4M ints (one wave
    // scatters a tile: small tiles give the scatter more waves)
    P.tile_tokens = NSA_IDX_MIN_TILE;
    while (div_up(P.T, P.tile_tokens) * (int64_t)P.nbc * P.Hkv > ((int64_t)1 << 22) && P.tile_tokens < (1 << 24))
        P.tile_tokens *= 2;
    P.ntiles = (int)div_up(P.T, P.tile_tokens);
    const bool half = d->dtype != NSA_SEL_DTYPE_F32;  // bf16 or fp16
    P.elt = half ? 2 : 4;
    const int64_t nbk = (int64_t)P.Hkv * P.nbc;
    const int64_t max_entries = P.T * P.Hkv * P.topk;
    P.item_rows = nsa::kItemRowsMax;
    while (P.item_rows > nsa::kItemRowsMin &&
           max_entries * P.G < (int64_t)nsa::kItemPlanPer * nsa::kItemPlanWgs * P.item_rows)
        P.item_rows /= 2;
    P.max_items = div_up(max_entries * P.G, P.item_rows) + nbk;

    size_t o = 0;
    P.o_status = o; o = align_up(o + sizeof(int32_t) * nsa::kStatusWords);
    P.o_cus = o; o = align_up(o + sizeof(int32_t) * (P.B + 1));
    P.o_blkoff = o; o = align_up(o + sizeof(int32_t) * (P.B + 1));
    P.o_tilecnt = o; o = align_up(o + sizeof(int32_t) * (size_t)P.Hkv * P.ntiles * P.nbc);
    P.o_counts = o; o = align_up(o + sizeof(int32_t) * (size_t)nbk);
    P.o_item_start = o; o = align_up(o + sizeof(int32_t) * (size_t)(nbk + 1));
    P.index_bytes = o;
    P.o_offsets = o; o = align_up(o + sizeof(int32_t) * (size_t)(nbk + 1));
    P.o_entries = o; o = align_up(o + sizeof(int32_t) * (size_t)max_entries);
    P.o_item_bucket = o; o = align_up(o + sizeof(int32_t) * (size_t)P.max_items);
    P.o_slot_pos = o; o = align_up(o + sizeof(int32_t) * (size_t)max_entries);
    P.o_dense_cnt = o; o = align_up(o + sizeof(int32_t) * (size_t)nbk);
    P.o_dense_ids = o; o = align_up(o + sizeof(int32_t) * (size_t)nbk * P.topk);
    if (half) {
        P.o_dense_lse = o; o = align_up(o + sizeof(float) * (size_t)P.T * P.Hq);
        P.o_dense_o = o; o = align_up(o + 2 * (size_t)P.T * P.Hq * P.D);
    } else {
        P.o_dense_lse = P.o_dense_o = 0;
    }
    P.o_part_lse = o; o = align_up(o + sizeof(float) * (size_t)max_entries * P.G);
    P.o_part_o = o; o = align_up(o + P.elt * (size_t)max_entries * P.G * P.D);
    P.fwd_bytes = o;

    o = P.o_entries + align_up(sizeof(int32_t) * (size_t)max_entries);
    P.o_bslot_pos = o; o = align_up(o + sizeof(int32_t) * (size_t)max_entries);
    P.o_delta = o; o = align_up(o + sizeof(float) * (size_t)P.T * P.Hq);
    P.o_dkv_part = o; o = align_up(o + sizeof(float) * 2 * (size_t)nsa::kBwdMaxGrid * 2 * P.bs * P.D);
    P.o_dq_part = o; o = align_up(o + 2 * (size_t)max_entries * P.G * P.D);
    P.bwd_bytes = o;
    return NSA_SEL_OK;
}

nsa::Params make_params(const Plan& P, const nsa_sel_desc* d, void* ws)
{
    nsa::Params p{};
    char* w = static_cast<char*>(ws);
    p.T = P.T;
    p.B = P.B; p.Hq = P.Hq; p.Hkv = P.Hkv; p.G = P.G; p.D = P.D; p.bs = P.bs; p.topk = P.topk;
    nsa::fast_div_init(P.G, p.g_mul, p.g_shr);
    nsa::fast_div_init(P.topk, p.topk_mul, p.topk_shr);
    p.nbc = P.nbc; p.ntiles = P.ntiles; p.tile_tokens = P.tile_tokens; p.item_rows = P.item_rows;
    p.flags = (int)d->flags;
    p.scale = d->scale;
    p.scale_log2 = d->scale * 1.4426950408889634f;
    p.max_items = P.max_items;
    p.status = reinterpret_cast<int32_t*>(w + P.o_status);
    p.cus = reinterpret_cast<int32_t*>(w + P.o_cus);
    p.blkoff = reinterpret_cast<int32_t*>(w + P.o_blkoff);
    p.tilecnt = reinterpret_cast<int32_t*>(w + P.o_tilecnt);
    p.counts = reinterpret_cast<int32_t*>(w + P.o_counts);
    p.item_start = reinterpret_cast<int32_t*>(w + P.o_item_start);
    return p;
}

thread_local char g_last_error[256] = "";

void set_error(const char* where, hipError_t e)
{
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%s)", where, hipGetErrorName(e),
             hipGetErrorString(e));
}

int hip_status(hipError_t e, const char* where)
{
    if (e == hipSuccess) return NSA_SEL_OK;
    set_error(where, e);
    return NSA_SEL_ERR_HIP;
}

// Clears an error left pending by earlier, unrelated HIP calls on this thread
// so that a failure reported afterwards is one of this library's launches.
void clear_stale_error()
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) set_error("pending before the call (cleared)", e);
    else g_last_error[0] = 0;
}

// Stage boundary i of a call: records the caller's event i on the call's
// stream when the descriptor carries stage events.
int mark(const nsa_sel_desc* d, int i, hipStream_t st)
{
    if (!d->stage_events || !d->stage_events[i]) return NSA_SEL_OK;
    return hip_status(hipEventRecord(static_cast<hipEvent_t>(d->stage_events[i]), st), "stage event record");
}

// Scratch of the allocation-free window forward: the status words, the
// sanitised cu_seqlens and the per-sequence block offsets that the window
// forward otherwise keeps in the caller's workspace.  Each GPU holds its own
// copy until the process ends; every call on a GPU shares it.
constexpr size_t kNoAllocScratchBytes = 64 << 10;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device
// (the array's name is only a host-side stand-in).
int scratch_ptr(void** out)
{
    int dev = -1;
    int rc = hip_status(hipGetDevice(&dev), "current device");
    if (rc != NSA_SEL_OK) return rc;
    if (dev < 0 || dev >= kMaxDevices) return NSA_SEL_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        rc = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "scratch address");
        if (rc != NSA_SEL_OK) return rc;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return NSA_SEL_OK;
}

}  // namespace

extern "C" {

int nsa_sel_version(void) { return NSA_SEL_ABI_VERSION; }

const char* nsa_sel_status_string(int status)
{
    switch (status) {
    case NSA_SEL_OK: return "ok";
    case NSA_SEL_ERR_INVALID_ARG: return "invalid argument";
    case NSA_SEL_ERR_UNSUPPORTED: return "unsupported configuration";
    case NSA_SEL_ERR_WORKSPACE: return "workspace missing or too small";
    case NSA_SEL_ERR_HIP: return "HIP runtime error";
    case NSA_SEL_ERR_BAD_INPUT: return "malformed cu_seqlens or block ids seen on device";
    default: return "unknown status";
    }
}

int nsa_sel_validate(const nsa_sel_desc* desc) { return check_desc(desc); }

const char* nsa_sel_last_error(void) { return g_last_error; }

int nsa_sel_index_sizes(const nsa_sel_desc* desc, int64_t* num_buckets, int64_t* max_entries)
{
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    if (num_buckets) *num_buckets = (int64_t)P.Hkv * P.nbc;
    if (max_entries) *max_entries = P.T * P.Hkv * P.topk;
    return NSA_SEL_OK;
}

int nsa_sel_index_workspace_size(const nsa_sel_desc* desc, size_t* bytes)
{
    if (!bytes) return NSA_SEL_ERR_INVALID_ARG;
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    *bytes = P.index_bytes;
    return NSA_SEL_OK;
}

int nsa_sel_fwd_workspace_size(const nsa_sel_desc* desc, size_t* bytes)
{
    if (!bytes) return NSA_SEL_ERR_INVALID_ARG;
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    *bytes = P.fwd_bytes;
    return NSA_SEL_OK;
}

int nsa_sel_workspace_size(const nsa_sel_desc* desc, size_t* bytes) { return nsa_sel_fwd_workspace_size(desc, bytes); }

int nsa_sel_build_index(const nsa_sel_desc* desc, const int32_t* cu_seqlens, const int32_t* block_idx,
                        int32_t* offsets, int32_t* entries, void* workspace, size_t workspace_bytes,
                        void* stream)
{
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    if (!cu_seqlens || !offsets || (P.T > 0 && (!block_idx || !entries))) return NSA_SEL_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < P.index_bytes) return NSA_SEL_ERR_WORKSPACE;
    nsa::Params p = make_params(P, desc, workspace);
    p.cu = cu_seqlens;
    p.block_idx = block_idx;
    p.offsets = offsets;
    p.entries = entries;
    clear_stale_error();
    return hip_status(nsa::launch_index(p, offsets, entries, static_cast<hipStream_t>(stream)),
                      "index inversion");
}

// The forward, after the inversion (offsets_in null) or on a prebuilt index.
static int run_fwd(const nsa_sel_desc* desc, const void* q, const void* k, const void* v,
                   const int32_t* cu_seqlens, const int32_t* block_idx, const int32_t* offsets_in,
                   const int32_t* entries_in, void* out, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream)
{
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    if (!cu_seqlens || (P.T > 0 && (!q || !k || !v || !block_idx || !out || !lse)))
        return NSA_SEL_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < P.fwd_bytes) return NSA_SEL_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(workspace);
    const int kind = elem_kind(desc->dtype);
    const bool half = kind != nsa::kElemF32;
    nsa::Params p = make_params(P, desc, workspace);
    p.cu = cu_seqlens;
    p.block_idx = block_idx;
    p.q = q; p.k = k; p.v = v;
    p.out = out;
    p.lse = lse;
    p.offsets = reinterpret_cast<int32_t*>(w + P.o_offsets);
    p.entries = reinterpret_cast<int32_t*>(w + P.o_entries);
    p.item_bucket = reinterpret_cast<int32_t*>(w + P.o_item_bucket);
    p.slot_pos = reinterpret_cast<int32_t*>(w + P.o_slot_pos);
    if (half && (desc->flags & NSA_SEL_FLAG_DENSE_SPLIT)) {
        // blocks kept by a whole token block go to the dense kernel
        p.dense_cnt = reinterpret_cast<int32_t*>(w + P.o_dense_cnt);
        p.dense_ids = reinterpret_cast<int32_t*>(w + P.o_dense_ids);
        p.dense_o = w + P.o_dense_o;
        p.dense_lse = reinterpret_cast<float*>(w + P.o_dense_lse);
        // the dense kernel merges its tokens itself when a token's G heads
        // share one 16-row tile
        p.fuse_merge = 16 % P.G == 0;
    }
    if (half) p.main_grid = (int)std::min<int64_t>(nsa::main_grid_size(P.D, P.bs, kind), div_up(P.max_items, 8) * 8);
    p.part_lse = reinterpret_cast<float*>(w + P.o_part_lse);
    p.part_o = w + P.o_part_o;
    clear_stale_error();
    if ((rc = mark(desc, 0, st)) != NSA_SEL_OK) return rc;
    if (offsets_in)
        rc = hip_status(nsa::launch_index_prebuilt(p, offsets_in, entries_in, (int)(P.T * P.Hkv * P.topk), st),
                        "prebuilt index");
    else
        rc = hip_status(nsa::launch_index(p, p.offsets, p.entries, st), "index inversion");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 1, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_main(p, kind, st), "main kernel");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 2, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_dense(p, kind, st), "dense kernel");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 3, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_merge(p, kind, st), "merge kernel");
    if (rc == NSA_SEL_OK) rc = mark(desc, 4, st);
    return rc;
}

int nsa_sel_attn_fwd(const nsa_sel_desc* desc, const void* q, const void* k, const void* v,
                     const int32_t* cu_seqlens, const int32_t* block_idx, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    return run_fwd(desc, q, k, v, cu_seqlens, block_idx, nullptr, nullptr, out, lse, workspace, workspace_bytes,
                   stream);
}

int nsa_sel_attn_fwd_indexed(const nsa_sel_desc* desc, const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens, const int32_t* block_idx, const int32_t* offsets,
                             const int32_t* entries, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream)
{
    const int rc = check_desc(desc);
    if (rc != NSA_SEL_OK) return rc;
    if (desc->flags & NSA_SEL_FLAG_DENSE_SPLIT) return NSA_SEL_ERR_UNSUPPORTED;
    if (!offsets || (desc->total_tokens > 0 && !entries)) return NSA_SEL_ERR_INVALID_ARG;
    return run_fwd(desc, q, k, v, cu_seqlens, block_idx, offsets, entries, out, lse, workspace, workspace_bytes,
                   stream);
}

int nsa_sel_bwd_workspace_size(const nsa_sel_desc* desc, size_t* bytes)
{
    if (!bytes) return NSA_SEL_ERR_INVALID_ARG;
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    if (desc->dtype == NSA_SEL_DTYPE_F32) return NSA_SEL_ERR_UNSUPPORTED;
    // d = 256 with 128-key blocks: one workgroup would need 16 waves (a key
    // group per wave and two halves of d) at 4 waves per SIMD, fewer
    // registers than the backward kernel's K, V and dK / dV tiles take
    if (desc->head_dim == 256 && desc->block_size > 64) return NSA_SEL_ERR_UNSUPPORTED;
    *bytes = P.bwd_bytes;
    return NSA_SEL_OK;
}

int nsa_sel_attn_bwd(const nsa_sel_desc* desc, const void* q, const void* k, const void* v,
                     const void* out, const float* lse, const void* dout, const int32_t* cu_seqlens,
                     const int32_t* block_idx, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, void* stream)
{
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    if (desc->dtype == NSA_SEL_DTYPE_F32) return NSA_SEL_ERR_UNSUPPORTED;
    // d = 256 with 128-key blocks: one workgroup would need 16 waves (a key
    // group per wave and two halves of d) at 4 waves per SIMD, fewer
    // registers than the backward kernel's K, V and dK / dV tiles take
    if (desc->head_dim == 256 && desc->block_size > 64) return NSA_SEL_ERR_UNSUPPORTED;
    if (desc->flags != 0) return NSA_SEL_ERR_INVALID_ARG;
    if (!cu_seqlens || (P.T > 0 && (!q || !k || !v || !out || !lse || !dout || !block_idx || !dq ||
                                    !dk || !dv)))
        return NSA_SEL_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < P.bwd_bytes) return NSA_SEL_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(workspace);
    nsa::Params p = make_params(P, desc, workspace);
    p.cu = cu_seqlens;
    p.block_idx = block_idx;
    p.q = q; p.k = k; p.v = v;
    p.out = const_cast<void*>(out);
    p.lse = const_cast<float*>(lse);
    p.dout = dout;
    p.dq = dq; p.dk = dk; p.dv = dv;
    p.offsets = reinterpret_cast<int32_t*>(w + P.o_offsets);
    p.entries = reinterpret_cast<int32_t*>(w + P.o_entries);
    p.slot_pos = reinterpret_cast<int32_t*>(w + P.o_bslot_pos);
    p.delta = reinterpret_cast<float*>(w + P.o_delta);
    p.dkv_part = reinterpret_cast<float*>(w + P.o_dkv_part);
    p.dq_part = w + P.o_dq_part;
    const int kind = elem_kind(desc->dtype);
    p.bwd_grid = nsa::bwd_grid_size(P.D, P.bs, kind);
    clear_stale_error();
    if ((rc = mark(desc, 0, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_index(p, p.offsets, p.entries, st), "index inversion");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 1, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_bwd_delta(p, kind, st), "backward delta kernel");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 2, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_bwd_main(p, kind, st), "backward main kernel");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 3, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_bwd_dq_merge(p, kind, st), "backward dk/dv finish and dq merge kernels");
    if (rc == NSA_SEL_OK) rc = mark(desc, 4, st);
    return rc;
}

int nsa_sel_window_workspace_size(const nsa_sel_desc* desc, size_t* bytes)
{
    if (!bytes) return NSA_SEL_ERR_INVALID_ARG;
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    if (desc->dtype == NSA_SEL_DTYPE_F32) return NSA_SEL_ERR_UNSUPPORTED;
    *bytes = P.o_tilecnt;  // status words, sanitised cu_seqlens, block offsets
    return NSA_SEL_OK;
}

namespace {
// Workspace of the index producer: the status words, sanitised cu_seqlens and
// block offsets of the plan, then window and tile offsets and the compressed
// keys.
struct SelPlan {
    size_t o_cbase, o_tbase, o_order, o_kcmp, bytes;
    int cap;
};
SelPlan sel_plan(const Plan& P)
{
    SelPlan S;
    S.cap = nsa::select_cap(P.T, P.B);
    size_t o = P.o_tilecnt;
    S.o_cbase = o; o = align_up(o + sizeof(int32_t) * (size_t)(P.B + 1));
    S.o_tbase = o; o = align_up(o + sizeof(int32_t) * (size_t)(P.B + 1));
    // dispatch order of the token tiles (at most T / tokens-per-tile + B tiles)
    S.o_order = o; o = align_up(o + sizeof(int32_t) * (size_t)nsa::select_max_tiles(P.T, P.B, P.G));
    S.o_kcmp = o; o = align_up(o + 2 * (size_t)S.cap * P.Hkv * P.D);
    S.bytes = o;
    return S;
}
}  // namespace

int nsa_sel_select_workspace_size(const nsa_sel_desc* desc, size_t* bytes)
{
    if (!bytes) return NSA_SEL_ERR_INVALID_ARG;
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    if (desc->dtype == NSA_SEL_DTYPE_F32) return NSA_SEL_ERR_UNSUPPORTED;
    *bytes = sel_plan(P).bytes;
    return NSA_SEL_OK;
}

int nsa_sel_select_blocks(const nsa_sel_desc* desc, int kernel_size, int kernel_stride, int init_blocks,
                          int local_blocks, const void* q, const void* k, const int32_t* cu_seqlens,
                          int32_t* block_idx, void* workspace, size_t workspace_bytes, void* stream)
{
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    if (desc->dtype == NSA_SEL_DTYPE_F32) return NSA_SEL_ERR_UNSUPPORTED;
    if (desc->flags != 0 || kernel_size < 1 || kernel_stride < 1 || init_blocks < 0 || local_blocks < 0)
        return NSA_SEL_ERR_INVALID_ARG;
    if (!nsa::select_supported(P.D, P.G, P.bs, kernel_size, kernel_stride)) return NSA_SEL_ERR_UNSUPPORTED;
    if (!cu_seqlens || (P.T > 0 && (!q || !k || !block_idx))) return NSA_SEL_ERR_INVALID_ARG;
    const SelPlan S = sel_plan(P);
    if (!workspace || workspace_bytes < S.bytes) return NSA_SEL_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(workspace);
    nsa::Params p = make_params(P, desc, workspace);
    p.cu = cu_seqlens;
    p.q = q; p.k = k;
    p.sel_init = init_blocks;
    p.sel_local = local_blocks;
    p.sel_cap = S.cap;
    p.sel_tok = nsa::select_tokens(P.G, P.topk, init_blocks, local_blocks);
    p.sel_cbase = reinterpret_cast<int32_t*>(w + S.o_cbase);
    p.sel_tbase = reinterpret_cast<int32_t*>(w + S.o_tbase);
    p.sel_kcmp = w + S.o_kcmp;
    p.sel_out = block_idx;
    const int kind = elem_kind(desc->dtype);
    clear_stale_error();
    if ((rc = mark(desc, 0, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_prep(p, st), "sequence prep");
    if (rc == NSA_SEL_OK) rc = hip_status(nsa::launch_sel_prep(p, st), "window offsets");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 1, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_compress(p, kind, st), "compressed keys");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 2, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_select(p, kind, reinterpret_cast<int32_t*>(w + S.o_order), st), "block lists");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 3, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_sel_orphans(p, st), "lists outside every sequence");
    if (rc == NSA_SEL_OK) rc = mark(desc, 4, st);
    return rc;
}

int nsa_sel_window_fwd(const nsa_sel_desc* desc, int window, const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream)
{
    Plan P;
    int rc = make_plan(desc, &P);
    if (rc != NSA_SEL_OK) return rc;
    if (desc->dtype == NSA_SEL_DTYPE_F32) return NSA_SEL_ERR_UNSUPPORTED;
    if (desc->flags != 0 || window < 1) return NSA_SEL_ERR_INVALID_ARG;
    if (!cu_seqlens || (P.T > 0 && (!q || !k || !v || !out || !lse))) return NSA_SEL_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < P.o_tilecnt) return NSA_SEL_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    nsa::Params p = make_params(P, desc, workspace);
    p.cu = cu_seqlens;
    p.q = q; p.k = k; p.v = v;
    p.out = out;
    p.lse = lse;
    p.window = window;
    const int kind = elem_kind(desc->dtype);
    clear_stale_error();
    if ((rc = mark(desc, 0, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_prep(p, st), "sequence prep");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 1, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_window(p, kind, st), "window kernel");
    if (rc != NSA_SEL_OK) return rc;
    if ((rc = mark(desc, 2, st)) != NSA_SEL_OK) return rc;
    rc = hip_status(nsa::launch_window_orphans(p, kind, st), "window orphan rows");
    if (rc == NSA_SEL_OK) rc = mark(desc, 3, st);
    if (rc == NSA_SEL_OK) rc = mark(desc, 4, st);
    return rc;
}

int nsa_sel_window_fwd_noalloc(const nsa_sel_desc* desc, int window, const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens, void* out, float* lse, void* stream)
{
    size_t need = 0;
    int rc = nsa_sel_window_workspace_size(desc, &need);
    if (rc != NSA_SEL_OK) return rc;
    if (need > kNoAllocScratchBytes) return NSA_SEL_ERR_WORKSPACE;
    if (desc->flags != 0 || window < 1) return NSA_SEL_ERR_INVALID_ARG;
    if (!cu_seqlens || (desc->total_tokens > 0 && (!q || !k || !v || !out || !lse))) return NSA_SEL_ERR_INVALID_ARG;
    clear_stale_error();
    void* ws = nullptr;
    rc = scratch_ptr(&ws);
    if (rc != NSA_SEL_OK) return rc;
    // the window kernels' first launch (sequence prep) clears the status words
    return nsa_sel_window_fwd(desc, window, q, k, v, cu_seqlens, out, lse, ws, kNoAllocScratchBytes, stream);
}

int nsa_sel_check(const void* workspace, void* stream, int* device_status)
{
    if (!workspace || !device_status) return NSA_SEL_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc = hip_status(hipStreamSynchronize(st), "stream synchronise");
    if (rc != NSA_SEL_OK) return rc;
    int32_t word = 0;
    rc = hip_status(hipMemcpy(&word, static_cast<const char*>(workspace) + nsa::kStatusError * sizeof(int32_t),
                              sizeof(word), hipMemcpyDeviceToHost), "status read");
    if (rc != NSA_SEL_OK) return rc;
    *device_status = word;
    return word ? NSA_SEL_ERR_BAD_INPUT : NSA_SEL_OK;
}

}  // extern "C"
