/*
 * nsa_sel.h -- C ABI of the MI355X (gfx950) selected-block attention library.
 *
 * The operation is Native Sparse Attention's selection branch for prefill:
 * every query token attends, for each query head of its GQA group, only to
 * the keys of the blocks of `block_size` tokens that its row of the block
 * index names (Flash-Sparse-Attention project page, agentlenshq
 * "Relaxed-System-Lab/Flash-Sparse-Attention": "Quick start" for
 * block_size / topk and the cu_seqlens varlen packing, "Key features" for the
 * GQA-aware design and the forward-only prefill use; q2bstudio "FSA:
 * efficient implementation of native sparse attention", first paragraph, for
 * why small GQA groups matter).  The work is split the FSA way ("Key
 * features", optimised-kernels row: a main batched query-to-KV kernel, a
 * reduction and an online softmax, no atomics): an index inversion turns
 * per-token block lists into per-block token lists, a main kernel runs each
 * K/V block once against the gathered queries that chose it, and a merge
 * kernel combines the per-block partial results of every query.
 *
 * Definition (what every entry point computes).  Tokens of sequence s are
 * t = cu_seqlens[s] + i, 0 <= i < L_s, in block b(t) = i / block_size.
 * For kv head h the selected set of row (t, h) is the set of distinct ids
 * j in block_idx[t][h][0..topk) with 0 <= j <= b(t); -1 (anywhere in the
 * row), future blocks and repeats add nothing, and the first position of j
 * in the row is its slot.  The keys of (t, h) are the positions p of the
 * selected blocks with p < L_s and p <= i.  Query head qh uses kv head
 * qh / G, G = num_q_heads / num_kv_heads.  With s_p = scale * q . k_p:
 *   out[t][qh] = sum_p softmax(s)_p v_p,  lse[t][qh] = ln sum_p exp(s_p),
 * and a row with no keys gives out = 0, lse = -inf.
 *
 * Conventions.
 *  - All tensor pointers are DEVICE pointers, dense row-major, 16-byte
 *    aligned, owned by the caller.  The library never allocates or frees
 *    device memory and keeps no pointer after a call returns.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream).  No entry point synchronises the stream except
 *    nsa_sel_check.  Calls that share a workspace must not overlap.
 *  - Every entry point returns an nsa_sel_status.  Argument errors are
 *    detected on the host before anything is enqueued; nothing is written
 *    then.
 *  - Malformed device data (cu_seqlens not running 0..T non-decreasingly,
 *    block ids < -1 or >= the sequence's block count) never causes an
 *    out-of-bounds access: cu_seqlens is read as its running maximum
 *    clamped to [0, T], such ids are ignored, and tokens outside
 *    [cu_seqlens[0], cu_seqlens[B]) get out = 0, lse = -inf.  The kernels
 *    record what they saw in the workspace; nsa_sel_check reads it.
 */
#ifndef NSA_SEL_H
#define NSA_SEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NSA_SEL_ABI_VERSION 2

typedef enum nsa_sel_status {
    NSA_SEL_OK = 0,
    NSA_SEL_ERR_INVALID_ARG = -1,   /* null pointer, bad shape, Hq % Hkv != 0 */
    NSA_SEL_ERR_UNSUPPORTED = -2,   /* dtype / head_dim / block_size / topk / size limit */
    NSA_SEL_ERR_WORKSPACE = -3,     /* workspace missing or too small */
    NSA_SEL_ERR_HIP = -4,           /* a HIP launch or runtime call failed */
    NSA_SEL_ERR_BAD_INPUT = -5      /* nsa_sel_check: malformed device data seen */
} nsa_sel_status;

typedef enum nsa_sel_dtype {
    NSA_SEL_DTYPE_BF16 = 1,         /* q, k, v, out bfloat16; fp32 accumulation */
    NSA_SEL_DTYPE_F32 = 2,          /* q, k, v, out float32 */
    NSA_SEL_DTYPE_F16 = 3           /* q, k, v, out float16 (IEEE half); fp32 accumulation */
} nsa_sel_dtype;

/*
 * Problem descriptor.  Supported: dtype BF16, F16 or F32; head_dim 64 or 128,
 * or 256 with BF16 / F16 (the pages' implementation takes one shared head dim
 * of at most 256: Flash-Sparse-Attention project page, "Limitations / future
 * plans"); the backward takes BF16 / F16, at head_dim 256 block_size <= 64;
 * block_size 32, 64 or 128; 1 <= topk <= 64; num_q_heads a multiple of
 * num_kv_heads with G <= 64; total_tokens * num_q_heads * topk < 2^31 and
 * (total_tokens / block_size + num_seqs) * num_kv_heads < 2^31 (the index's
 * 32-bit entries and bucket ids).  Sequences of any length within those.
 * Anything else returns NSA_SEL_ERR_UNSUPPORTED (or INVALID_ARG for shapes
 * that make no sense).
 */
typedef struct nsa_sel_desc {
    uint32_t struct_size;   /* sizeof(nsa_sel_desc) */
    int32_t dtype;          /* nsa_sel_dtype */
    int32_t num_seqs;       /* B >= 1 */
    int32_t num_q_heads;    /* Hq */
    int64_t total_tokens;   /* T >= 0 (= cu_seqlens[B]) */
    int32_t num_kv_heads;   /* Hkv */
    int32_t head_dim;       /* d, shared by q, k and v */
    int32_t block_size;     /* bs */
    int32_t topk;           /* slots per row of block_idx */
    float scale;            /* score scale, usually 1/sqrt(d) */
    uint32_t flags;         /* NSA_SEL_FLAG_* bits; other bits must be 0 */
    /* Stage timing (diagnostics; NULL for none): an array of
     * NSA_SEL_STAGE_EVENTS hipEvent_t that the caller created and owns.  A
     * compute entry point records event i on its stream at the start of its
     * stage i and the last one after its last stage; the caller reads the
     * stage durations with hipEventElapsedTime.  Stages -- forward: index
     * inversion, main kernel, dense kernel (empty without the dense split;
     * with it and a GQA group size dividing 16 it also merges every token of
     * a sequence), merge (in that fused form only the rows of tokens outside
     * every sequence).  Backward: index inversion, delta, main kernel, dk/dv
     * finish with the dq merge.  Window: sequence prep, window kernel, rows
     * outside every sequence, (empty).  Index producer: sequence and window
     * offsets, compressed keys, block lists, rows outside every sequence.
     * Host-only entry points ignore it.  The library keeps no state between
     * calls: nothing about the events outlives the call. */
    void *const *stage_events;
} nsa_sel_desc;

/* Events a call records when desc->stage_events is set: four stages. */
#define NSA_SEL_STAGE_EVENTS 5

/*
 * Dense split (BF16 and F16; ignored for F32): the blocks that every token of a
 * token block keeps are computed for the whole token block at once by a
 * dense kernel instead of once per token through the gather path and the
 * per-slot partials.  The result is the same up to rounding.  Off unless
 * set; on the 64K+32K GQA-4 workload it is the faster form (about 6.5 ms
 * against 6.9 ms without it on MI355X).
 */
#define NSA_SEL_FLAG_DENSE_SPLIT 1u

/* ABI version (NSA_SEL_ABI_VERSION). */
int nsa_sel_version(void);

/* Static description of a status code; never NULL. */
const char *nsa_sel_status_string(int status);

/*
 * Detail of the last NSA_SEL_ERR_HIP returned on the calling thread: which
 * stage failed and the HIP error name and text.  Empty when the last call on
 * this thread succeeded.  The string is owned by the library (thread-local).
 */
const char *nsa_sel_last_error(void);

/* Host-only check of a descriptor (no GPU needed). */
int nsa_sel_validate(const nsa_sel_desc *desc);

/*
 * Host-only sizes of the inverted index for `desc`:
 *   *num_buckets = num_kv_heads * (total_tokens / block_size + num_seqs)
 *     (offsets holds num_buckets + 1 int32),
 *   *max_entries = total_tokens * num_kv_heads * topk (capacity of entries).
 * Either output pointer may be NULL.
 */
int nsa_sel_index_sizes(const nsa_sel_desc *desc, int64_t *num_buckets,
                        int64_t *max_entries);

/* Host-only workspace bytes needed by nsa_sel_build_index. */
int nsa_sel_index_workspace_size(const nsa_sel_desc *desc, size_t *bytes);

/*
 * Index inversion alone: per-row block lists -> per-block token lists (CSR).
 * Bucket of a kept (t, h, j) is h * NBC + blkoff[s] + j, where
 * NBC = total_tokens / block_size + num_seqs and blkoff[s] counts the blocks
 * (ceil(L / block_size)) of the sequences before s.  Bucket lists hold
 * t * topk + slot, ascending in t; offsets[bkt] is the exclusive prefix sum
 * of the bucket sizes (empty and unused buckets repeat it) and
 * offsets[num_buckets] = nnz.  The result is deterministic and unique.
 *   cu_seqlens int32 [B+1], block_idx int32 [T][Hkv][topk]  (device, in)
 *   offsets int32 [num_buckets+1], entries int32 [max_entries] (device, out)
 */
int nsa_sel_build_index(const nsa_sel_desc *desc, const int32_t *cu_seqlens,
                        const int32_t *block_idx, int32_t *offsets,
                        int32_t *entries, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Host-only workspace bytes needed by nsa_sel_attn_fwd and
 * nsa_sel_attn_fwd_indexed (an upper bound from the descriptor alone). */
int nsa_sel_fwd_workspace_size(const nsa_sel_desc *desc, size_t *bytes);
/* The same number under its short name. */
int nsa_sel_workspace_size(const nsa_sel_desc *desc, size_t *bytes);

/*
 * Selected-block attention forward (prefill):
 *   q [T][Hq][d], k and v [T][Hkv][d]   (dtype of desc; device, in)
 *   cu_seqlens int32 [B+1], block_idx int32 [T][Hkv][topk] (device, in)
 *   out [T][Hq][d] (dtype of desc), lse float32 [T][Hq] natural log (device, out)
 *   workspace: at least nsa_sel_fwd_workspace_size bytes of device memory.
 * Runs the inversion, the main kernel and the merge on `stream`.  The result
 * does not depend on the order of the ids within a row and is bitwise
 * reproducible from run to run.
 */
int nsa_sel_attn_fwd(const nsa_sel_desc *desc, const void *q, const void *k,
                     const void *v, const int32_t *cu_seqlens,
                     const int32_t *block_idx, void *out, float *lse,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * The forward on a prebuilt index, so that one inversion serves several
 * calls: offsets and entries are what nsa_sel_build_index wrote for the same
 * descriptor, cu_seqlens and block_idx (device, in; entries with room for
 * max_entries ints, see nsa_sel_index_sizes).  Instead of the inversion it
 * rebuilds the forward's work lists from them (one pass over the entries and
 * their rows), then runs the main kernel and the merge; the result is
 * bitwise that of nsa_sel_attn_fwd.  Other arguments as there.  The order
 * of the entries within a bucket does not matter (any order gives the same
 * result, bitwise).  An index
 * that does not match block_idx stays memory-safe: an entry that is not a
 * kept (t, slot) of its bucket is ignored and sets bit 8 of the status word
 * (nsa_sel_check), and a kept slot missing from the index is left out of its
 * row's result.  flags must not hold NSA_SEL_FLAG_DENSE_SPLIT
 * (NSA_SEL_ERR_UNSUPPORTED); null offsets, or null entries with
 * total_tokens > 0, give NSA_SEL_ERR_INVALID_ARG.
 *   workspace: at least nsa_sel_fwd_workspace_size bytes of device memory.
 */
int nsa_sel_attn_fwd_indexed(const nsa_sel_desc *desc, const void *q,
                             const void *k, const void *v,
                             const int32_t *cu_seqlens,
                             const int32_t *block_idx, const int32_t *offsets,
                             const int32_t *entries, void *out, float *lse,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/* Host-only workspace bytes needed by nsa_sel_attn_bwd (BF16 or F16). */
int nsa_sel_bwd_workspace_size(const nsa_sel_desc *desc, size_t *bytes);

/*
 * Selected-block attention backward (training; Flash-Sparse-Attention
 * project page, "Key features", training-and-inference row, and "Quick
 * start", step 4).  Gradients of a loss L given dout = dL/dout:
 *   P_p = exp(s_p - lse[t][qh]) over the keys p of row (t, h) (as in the
 *   forward), D = sum_e dout[t][qh][e] * out[t][qh][e],
 *   dS_p = P_p (dout[t][qh] . v_p - D),
 *   dq[t][qh] = scale * sum_p dS_p k_p,
 *   dk[p][h] = scale * sum of dS_p q[t][qh], dv[p][h] = sum of P_p dout[t][qh]
 *   over every (t, qh) whose keys include p.
 *   q, out, dout [T][Hq][d]; k, v [T][Hkv][d]   (dtype of desc; device, in)
 *   lse float32 [T][Hq]: the forward's lse   (device, in)
 *   cu_seqlens, block_idx as for nsa_sel_attn_fwd   (device, in)
 *   dq [T][Hq][d], dk and dv [T][Hkv][d]   (dtype of desc; device, out; every element
 *   is written: keys nobody attends to and tokens outside every sequence
 *   get 0)
 *   workspace: at least nsa_sel_bwd_workspace_size bytes of device memory.
 * dtype must be BF16 or F16 (F32 gives NSA_SEL_ERR_UNSUPPORTED) and flags 0.  dk
 * and dv are summed per kv block without atomics; the result does not depend
 * on the order of the ids within a row and is bitwise reproducible on a
 * given device.
 */
int nsa_sel_attn_bwd(const nsa_sel_desc *desc, const void *q, const void *k,
                     const void *v, const void *out, const float *lse,
                     const void *dout, const int32_t *cu_seqlens,
                     const int32_t *block_idx, void *dq, void *dk, void *dv,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Host-only workspace bytes needed by nsa_sel_window_fwd (BF16 or F16). */
int nsa_sel_window_workspace_size(const nsa_sel_desc *desc, size_t *bytes);

/* Host-only workspace bytes needed by nsa_sel_select_blocks (BF16 or F16). */
int nsa_sel_select_workspace_size(const nsa_sel_desc *desc, size_t *bytes);

/*
 * Index producer: the selection branch's block lists from compressed
 * attention, in the layout nsa_sel_attn_fwd takes (Flash-Sparse-Attention
 * project page, "Quick start", step 2: kernel_size, kernel_stride,
 * block_size, topk, init_blocks, local_blocks).  For a sequence of length L
 * and kv head h:
 *   - compressed key of window c (positions [c*stride, c*stride + ks),
 *     c < (L - ks) / stride + 1): the mean of the window's k rows, summed in
 *     fp32 in position order, rounded to the input format;
 *   - for token t at local position i and query head qh of the group of h:
 *     p = softmax over the windows with c*stride + ks - 1 <= i of
 *     scale * q[t][qh] . kc[c] (none visible: p = 0);
 *   - importance of block j: the sum over the group's query heads and over
 *     the visible windows that overlap [j*bs, (j+1)*bs) of p;
 *   - block_idx[t][h][:]: init blocks 0 .. init_blocks-1, then local blocks
 *     b, b-1, .., b-local_blocks+1 (b = i / bs; ids outside [0, b] or
 *     repeated skipped), then the other blocks of [0, b] by importance,
 *     largest first (ties: lower id), up to topk ids; -1 after them.  Tokens
 *     outside every sequence get -1 rows.
 *   q [T][Hq][d], k [T][Hkv][d]   (BF16 or F16; device, in)
 *   cu_seqlens int32 [B+1]   (device, in)
 *   block_idx int32 [T][Hkv][topk]   (device, out)
 *   Supported: kernel_size 32, kernel_stride 16, block_size 64, head_dim 64
 *   or 128, G = Hq / Hkv in {1, 2, 4, 8, 16}, init_blocks, local_blocks >= 0;
 *   flags must be 0.  Sequences of any length are taken (the lists keep a
 *   running top-k per token, no per-block table).
 *   workspace: at least nsa_sel_select_workspace_size bytes (the compressed
 *   keys: about T/16 * Hkv * d * 2 bytes).
 * The result is bitwise reproducible: every sum has a fixed order.
 */
int nsa_sel_select_blocks(const nsa_sel_desc *desc, int kernel_size, int kernel_stride,
                          int init_blocks, int local_blocks, const void *q, const void *k,
                          const int32_t *cu_seqlens, int32_t *block_idx, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Sliding-window branch forward (Flash-Sparse-Attention project page,
 * "Quick start", window_size: NSA's third branch beside compression and
 * selection).  Token t = cu_seqlens[s] + i attends, for every query head, to
 * the keys p of its own sequence with i - window < p <= i:
 *   out[t][qh] = sum_p softmax(s)_p v_p,  lse[t][qh] = ln sum_p exp(s_p),
 *   s_p = scale * q . k_p, query head qh using kv head qh / G.
 *   q [T][Hq][d], k and v [T][Hkv][d]   (BF16 or F16; device, in)
 *   cu_seqlens int32 [B+1]   (device, in)
 *   out [T][Hq][d] (dtype of desc), lse float32 [T][Hq]   (device, out;
 *   tokens outside every sequence get out = 0, lse = -inf)
 *   window >= 1; desc->block_size is the kernel's tile (32, 64 or 128);
 *   desc->topk is ignored; flags must be 0.
 *   workspace: at least nsa_sel_window_workspace_size bytes (a few KB).
 */
int nsa_sel_window_fwd(const nsa_sel_desc *desc, int window, const void *q,
                       const void *k, const void *v, const int32_t *cu_seqlens,
                       void *out, float *lse, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * The sliding-window forward without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and result as
 * nsa_sel_window_fwd, bitwise; the few words that call keeps in its workspace
 * (status, sanitised cu_seqlens, per-sequence block offsets) live instead in
 * a 64 KiB device array of the library, one per GPU, held until the process
 * ends.  Nothing is allocated: no hipMalloc, hipFree or allocating library
 * call; the array's address is looked up on the first call on each device
 * (the current device, which must be the one `stream` belongs to).
 * Limit: the problem's window workspace (nsa_sel_window_workspace_size) must
 * fit in 64 KiB, about num_seqs <= 8000; a larger one returns
 * NSA_SEL_ERR_WORKSPACE before anything is enqueued.  Every call on a GPU
 * shares the array, so calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.  Malformed-input bits
 * are kept in the array and cannot be read with nsa_sel_check.
 */
int nsa_sel_window_fwd_noalloc(const nsa_sel_desc *desc, int window, const void *q,
                               const void *k, const void *v, const int32_t *cu_seqlens,
                               void *out, float *lse, void *stream);

/*
 * Synchronises `stream`, then reads the malformed-input word that the last
 * nsa_sel_build_index, nsa_sel_attn_fwd, nsa_sel_attn_fwd_indexed,
 * nsa_sel_attn_bwd, nsa_sel_window_fwd or nsa_sel_select_blocks call left in
 * `workspace`.  *device_status gets its bits (1: cu_seqlens malformed, 2: a
 * block id < -1 or >= the sequence's block count, 8: a prebuilt index
 * entry that does not match block_idx); returns NSA_SEL_ERR_BAD_INPUT if any
 * is set, else NSA_SEL_OK.
 */
int nsa_sel_check(const void *workspace, void *stream, int *device_status);

#ifdef __cplusplus
}
#endif

#endif /* NSA_SEL_H */
