/*
 * pkv.h - paged-KV decode attention for AMD MI355X (gfx950): the C ABI.
 *
 * The operations follow three pages on KV-cache management:
 *   [P1] "Chapter 18 - KV-Cache Optimization Strategies" (Language Modelling -
 *        The Complete Guide), sections "How PagedAttention Works" (with the
 *        "Physical KV Block" figure), "Prefix Caching", "KV-Cache
 *        Quantization", "Token Eviction and Pruning".
 *   [P2] "KV Cache Engineering for LLM Serving, clearly explained", sections
 *        "The cache formula", 1 "GQA and MQA cache fewer heads", 3 "Sliding
 *        windows", 7 "Query-aware sparse reads", 8 "Quantization", 9
 *        "Eviction", 10 "Paging", 11 "Prefix reuse".
 *   [P3] Learning-AI topic t13_4 (KV cache management): block-table and
 *        copy-on-write paragraphs.
 *
 * Conventions (all entry points)
 * ------------------------------
 * Layout.  K and V caches are separate C-contiguous arrays
 *   k_cache, v_cache : [num_blocks][block_size][num_kv_heads][head_dim]
 * i.e. one physical block holds [block_size, n_kv_heads, d_k] keys and the
 * same for values ([P1] "Physical KV Block").  A flat slot number
 * slot = physical_block * block_size + offset names one row
 * cache[slot / block_size][slot % block_size][:][:] ([P3] block table).
 *   query, out      : [num_seqs][num_q_heads][head_dim]
 *   block_tables    : [num_seqs][max_blocks_per_seq] int32, row s maps logical
 *                     block i of sequence s to a physical block
 *   seq_lens        : [num_seqs] int32, tokens of each sequence that attention
 *                     reads (the newest token included)
 *   k_scales,
 *   v_scales        : [num_blocks][num_kv_heads] fp32, one scale per (physical
 *                     block, KV head), used only when the cache holds codes.
 * GQA: query head h reads KV head h / (num_q_heads / num_kv_heads) ([P2] s.1).
 *
 * Pointers.  Every tensor pointer is a DEVICE pointer unless the argument is
 * documented as host memory; the caller owns all memory.  No entry point
 * allocates device memory: scratch comes in through a caller-provided
 * workspace.  Integers in device arrays are int32.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Every device entry point only enqueues work on it and returns; it
 * never synchronises.
 *
 * Errors.  Every call returns a pkv_status.  Argument errors detectable on the
 * host return PKV_EINVAL / PKV_EUNSUPPORTED / PKV_EWORKSPACE before anything is
 * enqueued; a failed launch returns PKV_EHIP.  pkv_last_error() returns a
 * thread-local message for the last failing call on the calling thread.  No
 * C++ exception crosses this interface.
 *
 * Device-resident contents (block_tables, seq_lens, slot_mapping) are not
 * inspected on the fast path, because that would need a synchronisation.
 * Their preconditions:
 *   0 <= seq_lens[s] <= max_blocks_per_seq * block_size;
 *   block_tables[s][i] in [0, num_blocks) for i < ceil(seq_lens[s]/block_size)
 *     (later entries are never read);
 *   slot_mapping entries unique among non-negative ones and < num_blocks *
 *     block_size (negative = skip the token).
 * Kernels clamp out-of-range values so that a bad table never makes them
 * access memory outside the arrays, but the results are then unspecified.
 * pkv_validate_tables() checks the preconditions on host copies; setting the
 * environment variable PKV_CHECK=1 makes the device entry points copy the
 * arrays to the host, synchronise the stream and check them before launching.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_EINVAL = 1,       /* bad argument (shape, null pointer, value out of range) */
  PKV_EUNSUPPORTED = 2, /* dtype / head_dim / block_size / group combination not built */
  PKV_EWORKSPACE = 3,   /* workspace missing or smaller than required */
  PKV_EHIP = 4,         /* the HIP runtime reported an error */
  PKV_ENOMEM = 5        /* host block pool: no free block */
} pkv_status;

/* Storage types of query / cache / output elements. */
typedef enum pkv_dtype {
  PKV_F32 = 0,     /* IEEE binary32 */
  PKV_BF16 = 1,    /* bfloat16 */
  PKV_F16 = 2,     /* IEEE binary16 */
  PKV_I8 = 3,      /* signed 8-bit integer code, value = code * scale */
  PKV_FP8E4M3 = 4, /* OCP FP8 E4M3 ("fn": no inf, NaN = S.1111.111) code, value = code * scale */
  PKV_I4 = 5,      /* signed 4-bit integer code in -7..7, two per byte (element 2i in the low
                      nibble, 2i + 1 in the high nibble, two's complement); a cache row holds
                      head_dim / 2 bytes; value = code * scale */
  PKV_FP8E5M2 = 6  /* OCP FP8 E5M2 (bias 15; inf/NaN in the top exponent) code, value = code * scale */
} pkv_dtype;

/* Thread-local text of the last error on this thread ("" if none). */
const char* pkv_last_error(void);
/* Library version string. */
const char* pkv_version(void);

/* ------------------------------------------------------------------------ */
/* Decode attention                                                          */
/* ------------------------------------------------------------------------ */

/* Decode flags (bit set). */
enum {
  /* A hint: the blocks the decode reads are (nearly) all read by one
   * sequence of the batch only.  The caches are then read with the
   * non-temporal (streaming) load policy, so the stream does not evict data
   * that is reused; leave it off when many sequences share blocks, whose
   * reuse it would defeat.  For pkv_paged_attn_decode_shared_prefix it
   * concerns the blocks past the shared prefix, which that call reads apart.
   * Results are identical either way. */
  PKV_DECODE_STREAM_KV = 1
};

/*
 * Number of KV partitions per sequence for a given bound on the sequence
 * length: ceil(max_seq_len / partition_size).  partition_size 0 lets the
 * library choose for a cache of kv_dtype (see
 * pkv_paged_attn_partition_size); otherwise it must be a positive multiple
 * of block_size.  Returns 0 on bad arguments.
 */
int pkv_paged_attn_num_partitions(int kv_dtype, int max_seq_len, int block_size, int partition_size);

/*
 * The partition size (tokens) the library picks when the caller passes 0.
 * Partitions are the split granularity of the decode: a sequence's tokens
 * are cut only at multiples of partition_size.  For 16-bit and code caches
 * the decode numbers the partitions that hold a kept token across the whole
 * batch and gives every workgroup an equal run of them (a run may end
 * inside one sequence and continue over the next); a sequence cut over
 * several workgroups gets one partial result per piece, combined by
 * log-sum-exp.  The choice: one pass (a result >= max_seq_len, no partials)
 * up to 512 tokens; above, one block for 16-bit and code caches and 64
 * tokens for fp32 caches.
 */
int pkv_paged_attn_partition_size(int kv_dtype, int max_seq_len, int block_size);

/*
 * Bytes of scratch pkv_paged_attn_decode needs for a cache of kv_dtype.
 * Partial records each hold a query group's unnormalised accumulators
 * acc[G][head_dim], running maxima m[16] and softmax sums l[16] (G =
 * num_q_heads / num_kv_heads).  16-bit and code caches: 16 bytes per
 * sequence (rounded up to 256) for the split plan, then two records per
 * (workgroup, KV head); the workgroup count depends on the current device's
 * compute units.  fp32 caches: one record per (sequence, KV head,
 * partition).  0 when no sequence can be split.  max_seq_len must be
 * max_blocks_per_seq * block_size of the later call.
 */
size_t pkv_paged_attn_workspace_bytes(int kv_dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                                      int head_dim, int max_seq_len, int partition_size);

/*
 * Paged decode attention: one query token per sequence attends over the
 * sequence's cached keys and values, read block by block through its block
 * table ([P1] "How PagedAttention Works"; [P3] block table; [P2] s.10: the
 * blocks are read in logical order).  For every sequence s and query head h:
 *   out[s][h] = sum_t softmax_t(sm_scale * q[s][h] . K_s[t][kvh]) V_s[t][kvh]
 * over the kept positions t: all t < seq_lens[s]; with sink_tokens /
 * window_tokens not both 0, only t < sink_tokens or t >= seq_lens[s] -
 * window_tokens ([P1] "Token Eviction and Pruning": attention sinks plus a
 * recent window).  Scores accumulate in fp32; the result is rounded to
 * q_dtype (nearest even).  A sequence with no kept position gets zeros.
 *
 * q_dtype:  PKV_F32, PKV_BF16 or PKV_F16; out has the same dtype.
 * kv_dtype: equal to q_dtype, or a code type (PKV_I8, PKV_FP8E4M3,
 *           PKV_FP8E5M2, PKV_I4) with a bf16 or f16 query, dequantised in
 *           registers with k_scales / v_scales ([P2] s.8); k_scales /
 *           v_scales are ignored (may be NULL) otherwise.  PKV_I4 caches
 *           are built for head_dim 128.
 * head_dim: 64 or 128.  block_size: 16.  num_q_heads % num_kv_heads == 0.
 * partition_size: 0 = library's choice, else a positive multiple of
 *           block_size, at most 128 * min(num_kv_heads, 8) blocks for 16-bit
 *           and code caches: the split granularity (see
 *           pkv_paged_attn_partition_size).  A sequence split over several
 *           workgroups gets a partial record per piece in the workspace,
 *           and a merge kernel combines them by log-sum-exp; a sequence
 *           handled by one workgroup is written directly.
 *           16-bit and code caches also need num_seqs * max_blocks_per_seq
 *           < 2^29 (PKV_EUNSUPPORTED otherwise).
 * flags:    PKV_DECODE_* bits (0 for none); unknown bits give PKV_EINVAL.
 * workspace: device scratch of at least pkv_paged_attn_workspace_bytes(...)
 *           bytes, 128-byte aligned (may be NULL when that is 0).  Its
 *           contents on entry do not matter and are undefined on exit.
 * Calls on the same stream that share a workspace are ordered; calls on
 * different streams must not share one.
 */
pkv_status pkv_paged_attn_decode(
    void* out, const void* query, int q_dtype,
    const void* k_cache, const void* v_cache, int kv_dtype,
    const float* k_scales, const float* v_scales,
    const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* seq_lens, int num_seqs,
    int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
    float sm_scale, int partition_size, int sink_tokens, int window_tokens, unsigned flags,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same kernels and the same result,
 * bit for bit; the scratch (merge plan and partial records) is a fixed
 * device array of pkv_paged_attn_noalloc_scratch_bytes() bytes (64 MiB) that
 * the library holds on every GPU it runs on until the process ends.  The
 * call allocates nothing: no hipMalloc, no hipFree.
 * Errors: PKV_EWORKSPACE when pkv_paged_attn_workspace_bytes(...) for these
 * arguments exceeds that size (nothing is launched); otherwise as
 * pkv_paged_attn_decode.  The PKV_CHECK=1 host check is not run (it copies
 * the tables to the host); call pkv_validate_tables instead.
 * Every call on one GPU shares that GPU's array, and each call overwrites
 * what it needs before reading it: calls that overlap on one GPU (on
 * different streams, or from several threads) race and must not be issued.
 */
size_t pkv_paged_attn_noalloc_scratch_bytes(void);
pkv_status pkv_paged_attn_decode_noalloc(
    void* out, const void* query, int q_dtype,
    const void* k_cache, const void* v_cache, int kv_dtype,
    const float* k_scales, const float* v_scales,
    const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* seq_lens, int num_seqs,
    int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
    float sm_scale, int partition_size, int sink_tokens, int window_tokens, unsigned flags,
    void* stream);

/*
 * The two kernels pkv_paged_attn_decode launches, exposed so that each can be
 * timed on its own.  pkv_paged_attn_partition takes the same arguments and
 * writes the partials to the workspace (or `out` directly when one partition
 * covers max_blocks_per_seq * block_size); pkv_paged_attn_merge then combines
 * them into `out`.  Calling partition then merge on one stream with the same
 * arguments is exactly pkv_paged_attn_decode.  When no sequence can be
 * split, pkv_paged_attn_merge does nothing and returns PKV_OK.  For the
 * merge, max_seq_len is max_blocks_per_seq * block_size of the partition
 * call, and partition_size, sink_tokens and window_tokens must be the ones
 * the partition call used (they fix how the work was split).
 */
pkv_status pkv_paged_attn_partition(
    void* out, const void* query, int q_dtype,
    const void* k_cache, const void* v_cache, int kv_dtype,
    const float* k_scales, const float* v_scales,
    const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* seq_lens, int num_seqs,
    int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
    float sm_scale, int partition_size, int sink_tokens, int window_tokens, unsigned flags,
    void* workspace, size_t workspace_bytes, void* stream);

pkv_status pkv_paged_attn_merge(
    void* out, int q_dtype, const int32_t* seq_lens, int num_seqs,
    int num_q_heads, int num_kv_heads, int head_dim, int max_seq_len, int partition_size,
    int sink_tokens, int window_tokens,
    const void* workspace, size_t workspace_bytes, void* stream);

/*
 * Several new tokens per sequence at once (checking speculative drafts, or
 * a short chunk of prefill; the pages stop at one token per step, this is
 * the plain causal reading): query and out are [num_seqs][num_query_tokens]
 * [num_q_heads][head_dim]; seq_lens[s] = L counts the new tokens, whose
 * keys and values are already in the cache at positions L - T .. L - 1 (T =
 * num_query_tokens), and token t attends to positions 0 .. L - T + t.  One
 * pass over the cache serves all T tokens: T * (num_q_heads / num_kv_heads)
 * must be at most 16.  16-bit and code caches; no keep-mask.  The workspace
 * is pkv_paged_attn_workspace_bytes(kv_dtype, num_seqs, num_q_heads * T,
 * num_kv_heads, head_dim, max_blocks_per_seq * block_size, partition_size).
 * Other arguments as pkv_paged_attn_decode; T = 1 is that decode.
 */
pkv_status pkv_paged_attn_decode_multi(
    void* out, const void* query, int q_dtype,
    const void* k_cache, const void* v_cache, int kv_dtype,
    const float* k_scales, const float* v_scales,
    const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* seq_lens, int num_seqs, int num_query_tokens,
    int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
    float sm_scale, int partition_size, unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Query-aware page selection (Quest)                                        */
/* ------------------------------------------------------------------------ */
/*
 * [P2] s.7 "Query-aware sparse reads": each page keeps the minimum and the
 * maximum of its keys in every key dimension; a query scores a page by the
 * sum over dimensions of max(q_i * min_i, q_i * max_i), the largest q . k a
 * key inside the page's box can reach, and only the highest-scoring pages
 * are read.  Nothing is evicted.  Here a page is one physical block; with
 * GQA a page's score for a KV head is the largest over the group's query
 * heads, and pages are chosen per (sequence, KV head).
 */

/*
 * Page summaries of the key cache: k_summary[NB][num_kv_heads][2][head_dim]
 * in kv_dtype (bf16 or f16), minimum first, then maximum, over the rows a
 * block holds (tokens < seq_lens[s]; a partial last block summarises its
 * written rows only).  last_only = 0: every block of every sequence (after
 * a prefill); 1: each sequence's last block only (after a decode step's
 * slot write).  Blocks no sequence reaches are left alone.  A block shared
 * by several sequences gets the same summary from each.
 */
pkv_status pkv_quest_summarize(const void* k_cache, int kv_dtype, void* k_summary,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* seq_lens, int num_seqs, int num_blocks, int block_size,
                               int num_kv_heads, int head_dim, int last_only, void* stream);

/* Bytes of scratch pkv_quest_select needs (8 per (sequence, KV head, block)).
 * For tables up to 9216 blocks wide, after a call that did not keep every
 * page, scratch[s][h][lb] holds two uint32 order keys (larger float, larger
 * key: the bits of a non-negative value with the top bit set, of a negative
 * one inverted): a lower and an upper bound of block lb's score, each a
 * float32.  Wider tables hold the exact scores there instead. */
size_t pkv_quest_scratch_bytes(int num_seqs, int num_kv_heads, int max_blocks_per_seq);

/*
 * Scores every page of every (sequence, KV head) against the query group
 * (fp64; each product of two 16-bit values is exact; for tables up to 9216
 * blocks wide, bounds from a float32 pass first settle most pages and only
 * the others are scored in fp64, with the same result) and writes, for each
 * (s, kvh), the budget_blocks highest-scoring pages in logical order to
 * selected[S][num_kv_heads][budget_blocks][2] as (physical block, logical
 * block) int32 pairs.  Equal scores keep the lower logical block.  A
 * sequence of n <= budget_blocks blocks keeps all n (entries past n are
 * left alone).  query: [S][Hq][D] bf16 / f16, the cache's 16-bit type.
 * scratch: pkv_quest_scratch_bytes(...) bytes, 8-byte aligned.
 */
pkv_status pkv_quest_select(const void* query, int q_dtype, const void* k_summary,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* seq_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                            int head_dim, int block_size, int num_blocks, int budget_blocks,
                            int32_t* selected, void* scratch, size_t scratch_bytes, void* stream);

/*
 * Decode attention reading only the selected pages: for query head h of
 * sequence s, softmax attention over the tokens t < seq_lens[s] of the
 * first min(budget_blocks, ceil(seq_lens[s] / block_size)) entries of
 * selected[s][h / G] (as pkv_quest_select writes them, or any list of
 * distinct blocks of the sequence in logical order).  Other arguments as
 * pkv_paged_attn_decode; 16-bit and code caches.  The workspace is
 * pkv_paged_attn_workspace_bytes(kv_dtype, num_seqs, num_q_heads,
 * num_kv_heads, head_dim, budget_blocks * block_size, block_size) bytes.
 */
pkv_status pkv_paged_attn_decode_selected(
    void* out, const void* query, int q_dtype,
    const void* k_cache, const void* v_cache, int kv_dtype,
    const float* k_scales, const float* v_scales,
    const int32_t* selected, int budget_blocks,
    const int32_t* seq_lens, int num_seqs,
    int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
    float sm_scale, unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Cache writes                                                              */
/* ------------------------------------------------------------------------ */

/*
 * Slot of each new token: slot_mapping[j] = block_tables[s][p / block_size] *
 * block_size + p % block_size with s = seq_ids[j] (or j when seq_ids is
 * NULL) and p = positions[j] ([P3] block table; [P1] new tokens fill the
 * current block).  Bit-exact integer arithmetic.  A token whose sequence id
 * is outside [0, num_seqs), whose position is negative or past the table, or
 * whose table entry is outside [0, num_blocks) gets slot -1.
 * All arrays are device int32 of length num_tokens (block_tables as above).
 */
pkv_status pkv_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables,
                            int max_blocks_per_seq, const int32_t* seq_ids,
                            const int32_t* positions, int num_tokens, int num_seqs,
                            int block_size, int num_blocks, void* stream);

/*
 * The slot write ([P1] "How PagedAttention Works"; [P3] new entries are
 * appended as tokens are generated): for each token j with
 * slot_mapping[j] >= 0, copies key[j][:][:] into k_cache at that slot and
 * value[j][:][:] into v_cache.  key/value: [num_tokens][num_kv_heads][head_dim]
 * of `dtype`, which must equal the caches' dtype (PKV_F32, PKV_BF16, PKV_F16).
 * A bit copy.  Slots >= num_blocks * block_size are skipped.
 */
pkv_status pkv_reshape_and_cache(const void* key, const void* value,
                                 void* k_cache, void* v_cache, int dtype,
                                 const int32_t* slot_mapping, int num_tokens,
                                 int num_blocks, int block_size, int num_kv_heads,
                                 int head_dim, void* stream);

/*
 * pkv_slot_mapping and pkv_reshape_and_cache in one launch: token j (of
 * sequence seq_ids[j], or j when seq_ids is NULL, at position positions[j])
 * gets slot block_tables[s][p / block_size] * block_size + p % block_size
 * and its key[j] / value[j] rows are copied there.  A token whose slot would
 * be -1 under pkv_slot_mapping is skipped.  slot_mapping (device int32
 * [num_tokens]) receives the slots when not NULL.  Same layouts, dtypes and
 * bit-exactness as the two calls it combines; the same tokens must not map
 * to one slot.
 */
pkv_status pkv_append_kv(const void* key, const void* value, void* k_cache, void* v_cache, int dtype,
                         const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_ids,
                         const int32_t* positions, int32_t* slot_mapping, int num_tokens, int num_seqs,
                         int num_blocks, int block_size, int num_kv_heads, int head_dim, void* stream);

/*
 * Copy-on-write block duplication ([P3] copy-on-write: a shared block is
 * duplicated when a sequence diverges; [P1] "Prefix Caching"): for each pair
 * i, copies every slot and head of physical block src_dst[2i] onto block
 * src_dst[2i+1] in k_cache and v_cache, and, when k_scales / v_scales are not
 * NULL, their [num_kv_heads] scale rows.  src_dst is device int32 [n][2].
 * Pairs must not overlap (no block is both a destination and another pair's
 * source).  Indices outside [0, num_blocks) are skipped.  Bit copy.
 */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                           const int32_t* src_dst, int n, int dtype, int num_blocks,
                           int block_size, int num_kv_heads, int head_dim, void* stream);

/*
 * Symmetric absmax quantisation of whole cache blocks ([P2] s.8;
 * [P1] "KV-Cache Quantization"), one scale per (block, KV head) over its
 * [block_size, head_dim] tile:
 *   a = max |x|;  scale = fp32(a / qmax)  (IEEE division; qmax = 127 for
 *   PKV_I8, 7 for PKV_I4, 448 for PKV_FP8E4M3, 57344 for PKV_FP8E5M2);
 *   code = round_half_even(fp32(x / scale)) clipped to [-qmax, qmax]  (I8, I4)
 *   code = FP8 round-to-nearest-even of fp32(x / scale), saturating at
 *          +-qmax, sign of zero kept                                  (FP8)
 *   a == 0 gives scale 0 and all codes 0.
 * src_cache: [num_blocks][block_size][num_kv_heads][head_dim] of src_dtype
 * (PKV_F32, PKV_BF16, PKV_F16); dst_codes: the same shape in code_dtype
 * (PKV_I8, PKV_I4 - head_dim / 2 bytes per row -, PKV_FP8E4M3 or
 * PKV_FP8E5M2); dst_scales: [num_blocks][num_kv_heads] fp32.
 * block_ids: device int32 [n_blocks] of blocks to quantise, or NULL for
 * blocks 0..n_blocks-1.  Call once for K and once for V.  Every slot of a
 * quantised block must hold data.  Bit-exact.
 */
pkv_status pkv_quantize_kv(const void* src_cache, int src_dtype, void* dst_codes, int code_dtype,
                           float* dst_scales, const int32_t* block_ids, int n_blocks,
                           int num_blocks, int block_size, int num_kv_heads, int head_dim,
                           void* stream);

/*
 * pkv_paged_attn_decode with the step's slot write fused into it: for each
 * sequence s with positions[s] = p >= 0, key[s] / value[s]
 * ([num_seqs][num_kv_heads][head_dim] in the cache dtype) are written to
 * slot block_tables[s][p / block_size] * block_size + p % block_size, as
 * pkv_reshape_and_cache would, and the decode attends over seq_lens[s]
 * tokens with that row included.  The slot goes to slot_mapping_out[s] when
 * it is not NULL.  Precondition: p = seq_lens[s] - 1 (the new token is the
 * last one) and its block is in the table; the write is done by the
 * workgroup that reads that block, before it reads it, so with any other p
 * the attention may or may not see the new row.  Rows of sequences with
 * p < 0, or whose table entry is outside [0, num_blocks), are not written.
 * bf16 or f16 caches of the query dtype.  Workspace, partition_size,
 * sink_tokens / window_tokens (the keep-mask; the new row is written
 * whether or not the mask keeps it) and flags as in pkv_paged_attn_decode.
 * One launch fewer per decode step than pkv_append_kv followed by the
 * decode.
 */
pkv_status pkv_paged_attn_decode_append(void* out, const void* query, int q_dtype, void* k_cache, void* v_cache,
                                        int kv_dtype, const void* key, const void* value,
                                        const int32_t* positions, int32_t* slot_mapping_out,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* seq_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, int block_size, int num_blocks, float sm_scale,
                                        int partition_size, int sink_tokens, int window_tokens, unsigned flags,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode over a batch whose sequences all begin with the same prefix_blocks
 * physical blocks (a prompt stored once and shared through the block tables:
 * [P2] s.11 prefix reuse, [P1] "Prefix Caching", [P3] copy-on-write).  The
 * result is pkv_paged_attn_decode's (softmax attention of each query over
 * its seq_lens[s] tokens; the shared blocks are ordinary logical blocks
 * 0..prefix_blocks-1 of every sequence); only the order of the work
 * differs.  One pass attends every query row of the batch to the shared
 * blocks, reading each block once per 32 rows (a dense
 * [num_seqs * G, head_dim] x [head_dim, 16 * prefix_blocks] product on the
 * matrix cores), and leaves per (sequence, query head) fp32 acc[head_dim],
 * m, l at the start of the workspace.  The decode then reads each
 * sequence's blocks past the prefix and folds those records in by
 * log-sum-exp.
 * The shared blocks are sequence 0's first prefix_blocks table entries.
 * Preconditions (checked under PKV_CHECK=1, or by
 * pkv_validate_shared_prefix): every sequence has the same first
 * prefix_blocks entries and seq_lens[s] >= 16 * prefix_blocks; otherwise
 * the result is undefined (no access leaves the caches).  A sequence with
 * nothing past the prefix gets the prefix's attention.
 * key / value / positions / slot_mapping_out: optional fused slot write, as
 * in pkv_paged_attn_decode_append (key NULL: none; the new token must lie
 * past the prefix, a shared block is never written).
 * bf16 or f16 caches of the query dtype, head_dim 64 or 128, block_size 16,
 * query group size <= 16.  workspace: at least
 * pkv_paged_attn_shared_prefix_workspace_bytes bytes, 128-byte aligned;
 * partition_size and flags as in pkv_paged_attn_decode (they apply to the
 * blocks past the prefix).  Errors: PKV_EINVAL (bad sizes, null pointers,
 * prefix_blocks outside [1, max_blocks_per_seq]), PKV_EUNSUPPORTED (dtype,
 * head_dim, group size), PKV_EWORKSPACE, PKV_EHIP.
 */
pkv_status pkv_paged_attn_decode_shared_prefix(void* out, const void* query, int q_dtype, void* k_cache,
                                               void* v_cache, int kv_dtype, const void* key, const void* value,
                                               const int32_t* positions, int32_t* slot_mapping_out,
                                               const int32_t* block_tables, int max_blocks_per_seq,
                                               const int32_t* seq_lens, int num_seqs, int num_q_heads,
                                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                               float sm_scale, int prefix_blocks, int partition_size,
                                               unsigned flags, void* workspace, size_t workspace_bytes,
                                               void* stream);

/* Workspace bytes of pkv_paged_attn_decode_shared_prefix for sequences of
 * at most max_seq_len tokens (0 when num_seqs <= 0). */
size_t pkv_paged_attn_shared_prefix_workspace_bytes(int kv_dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                                                    int head_dim, int max_seq_len, int prefix_blocks,
                                                    int partition_size);

/* Host check of the shared-prefix preconditions on HOST copies of the
 * tables: every row's first prefix_blocks entries equal row 0's, and
 * seq_lens[s] >= prefix_blocks * block_size.  PKV_EINVAL with the first
 * violation in pkv_last_error(). */
pkv_status pkv_validate_shared_prefix(const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                                      int num_seqs, int block_size, int prefix_blocks);

/* Scale groups of the grouped quantiser and decode. */
typedef enum pkv_scale_group {
  PKV_GROUP_CHANNEL = 0, /* one scale per (block, KV head, channel) over the block's rows (keys) */
  PKV_GROUP_TOKEN = 1    /* one scale per (block, KV head, token row) over the channels (values) */
} pkv_scale_group;

/*
 * Absmax quantisation with grouped scales ([P2] s.8, the KIVI paragraph:
 * keys grouped by channel, values by token; here every group stays inside
 * one block tile).  Per (block, KV head) tile [block_size][head_dim], each
 * group g (a column for PKV_GROUP_CHANNEL, a row for PKV_GROUP_TOKEN) gets
 * scale_g = fp32(max |x_g| / qmax) and its elements the codes of
 * pkv_quantize_kv with that scale (qmax and rounding as there).
 * dst_codes: cache layout of code_dtype; dst_group_scales: fp32
 * [num_blocks][num_kv_heads][head_dim] (channel) or
 * [num_blocks][num_kv_heads][block_size] (token); dst_tile_scales: fp32
 * [num_blocks][num_kv_heads], each tile's largest group scale (the
 * one-scale tile rule's scale), or NULL to skip.  block_ids / n_blocks as
 * in pkv_quantize_kv.  Bit-exact.
 */
pkv_status pkv_quantize_kv_grouped(const void* src_cache, int src_dtype, void* dst_codes, int code_dtype,
                                   float* dst_tile_scales, float* dst_group_scales, int group,
                                   const int32_t* block_ids, int n_blocks, int num_blocks, int block_size,
                                   int num_kv_heads, int head_dim, void* stream);

/*
 * pkv_paged_attn_decode over a cache quantised with grouped scales: keys
 * by channel (k_channel_scales [num_blocks][num_kv_heads][head_dim] and
 * k_tile_scales [num_blocks][num_kv_heads] from pkv_quantize_kv_grouped
 * with PKV_GROUP_CHANNEL), values by token (v_token_scales
 * [num_blocks][num_kv_heads][block_size], PKV_GROUP_TOKEN).  A key is
 * code * channel scale, a value code * token scale.  kv_dtype PKV_I8
 * (head_dim 64 or 128) or PKV_I4 (head_dim 128); bf16 or f16 query; no
 * keep-mask.  The channel scales enter the products as f16 factors
 * scale / tile scale in (0, 1] (the tile scale joins the fp32 score
 * factor), so a channel below 2^-24 of its tile's largest reads as zero.
 * num_blocks * num_kv_heads < 2^25.  Workspace, partition_size and flags as
 * in pkv_paged_attn_decode (size it with the kv_dtype).
 */
pkv_status pkv_paged_attn_decode_grouped(void* out, const void* query, int q_dtype, const void* k_cache,
                                         const void* v_cache, int kv_dtype, const float* k_tile_scales,
                                         const float* k_channel_scales, const float* v_token_scales,
                                         const int32_t* block_tables, int max_blocks_per_seq,
                                         const int32_t* seq_lens, int num_seqs, int num_q_heads,
                                         int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                         float sm_scale, int partition_size, unsigned flags, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * Appends one token per sequence to a quantised cache (the pages leave the
 * how open; this is the reading taken).  Each sequence keeps the source
 * values of its partial last block in a tail, [num_seqs][block_size]
 * [num_kv_heads][head_dim] of src_dtype (caller-owned, one per K and V).
 * For sequence s with positions[s] = p >= 0: row p % block_size of its tail
 * takes key[s] / value[s] ([num_seqs][num_kv_heads][head_dim], src_dtype),
 * and block block_tables[s][p / block_size] is quantised again from the
 * tail's rows 0 .. p % block_size, the rows after them taken as zeros
 * ([P2] s.8 absmax rule, the arithmetic of pkv_quantize_kv): its codes and
 * its scales per KV head are rewritten, later rows get code 0.  Once a
 * block is full its codes and scales are exactly pkv_quantize_kv's for its
 * rows.  Tail rows before p % block_size must hold the block's earlier
 * tokens (a prefill's partial last block is copied into the tail by the
 * caller; a fork copies its parent's tail with the block).  positions[s] <
 * 0 skips sequence s; one token per sequence per call.
 */
pkv_status pkv_append_kv_quantized(const void* key, const void* value, int src_dtype,
                                   void* k_tail, void* v_tail, void* k_codes, void* v_codes,
                                   int code_dtype, float* k_scales, float* v_scales,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* positions, int num_seqs, int num_blocks, int block_size,
                                   int num_kv_heads, int head_dim, void* stream);

/*
 * pkv_append_kv_quantized for a cache with grouped scales (the layout of
 * pkv_quantize_kv_grouped): the block is quantised again from the tail with
 * keys scaled per channel (k_channel_scales [num_blocks][num_kv_heads]
 * [head_dim], their largest into k_tile_scales [num_blocks][num_kv_heads])
 * and values per token (v_token_scales [num_blocks][num_kv_heads]
 * [block_size]).  A token group depends on its own row only, so appending
 * leaves earlier rows' value codes and scales as they were.  Bit-exact.
 */
pkv_status pkv_append_kv_quantized_grouped(const void* key, const void* value, int src_dtype,
                                           void* k_tail, void* v_tail, void* k_codes, void* v_codes,
                                           int code_dtype, float* k_tile_scales, float* k_channel_scales,
                                           float* v_token_scales, const int32_t* block_tables,
                                           int max_blocks_per_seq, const int32_t* positions, int num_seqs,
                                           int num_blocks, int block_size, int num_kv_heads, int head_dim,
                                           void* stream);

/* ------------------------------------------------------------------------ */
/* Host-side checks                                                          */
/* ------------------------------------------------------------------------ */

/*
 * Checks the device-array preconditions listed above on HOST copies:
 * block_tables [num_seqs][max_blocks_per_seq], seq_lens [num_seqs] and,
 * when not NULL, slot_mapping [num_tokens].  Returns PKV_EINVAL with a
 * message naming the first violation.
 */
pkv_status pkv_validate_tables(const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* seq_lens, int num_seqs, int block_size,
                               int num_blocks, const int32_t* slot_mapping, int num_tokens);

/* ------------------------------------------------------------------------ */
/* Host block pool ([P2] s.10 free list; [P1] on-demand blocks; [P3] CoW)    */
/* ------------------------------------------------------------------------ */

/*
 * A pool of physical block ids with a FIFO free list and a reference count
 * per block.  Host memory only; not thread-safe (one owner thread).
 */
typedef struct pkv_pool pkv_pool;

/* Creates a pool of num_blocks blocks.  initial_order (host, may be NULL =
 * 0..num_blocks-1) gives the initial free-list order and must be a
 * permutation.  Returns NULL on bad arguments (see pkv_last_error). */
pkv_pool* pkv_pool_create(int num_blocks, const int32_t* initial_order);
void pkv_pool_destroy(pkv_pool* pool);

/* Takes the block at the front of the free list; its count becomes 1.
 * PKV_ENOMEM when the list is empty. */
pkv_status pkv_pool_alloc(pkv_pool* pool, int32_t* block_out);
/* Adds a reference to a block in use (sharing, e.g. a forked sequence). */
pkv_status pkv_pool_incref(pkv_pool* pool, int32_t block);
/* Drops a reference; a block whose count reaches 0 goes to the back of the
 * free list.  PKV_EINVAL for a free block. */
pkv_status pkv_pool_decref(pkv_pool* pool, int32_t block);
/* Reference count of a block (0 = free, -1 = out of range). */
int32_t pkv_pool_refcount(const pkv_pool* pool, int32_t block);

/*
 * Sequence-level operations ([P2] s.10 free-list example; [P1] "Prefix
 * Caching"; [P3] copy-on-write), each all-or-nothing: on an error nothing
 * changes.
 * pkv_pool_allocate_sequence: blocks for a new sequence of num_tokens tokens,
 *   ceil(num_tokens / block_size) of them taken from the front of the free
 *   list in order into table_out[0 .. *n_out).  PKV_ENOMEM if too few are
 *   free, PKV_EINVAL if table_capacity is smaller.
 * pkv_pool_fork: a new sequence shares every block of table[0 .. n): each
 *   gains one reference.  PKV_EINVAL if an entry is free or out of range.
 * pkv_pool_release: a finished sequence drops one reference per entry of
 *   table[0 .. n), in table order; blocks reaching 0 go to the back of the
 *   free list in that order.  PKV_EINVAL if an entry is free, out of range,
 *   or listed more often than it is referenced.
 */
pkv_status pkv_pool_allocate_sequence(pkv_pool* pool, int32_t num_tokens, int block_size,
                                      int32_t* table_out, int32_t table_capacity, int32_t* n_out);
pkv_status pkv_pool_fork(pkv_pool* pool, const int32_t* table, int32_t n);
pkv_status pkv_pool_release(pkv_pool* pool, const int32_t* table, int32_t n);

/*
 * Reserves the slot of token number seq_len of a sequence whose host table
 * table[0 .. *table_len) covers seq_len tokens.  If seq_len % block_size == 0
 * a new block is appended to the table (table_capacity bounds it).
 * Otherwise, if the current last block is shared (count > 1), a new block is
 * taken, the old block loses one reference and the table entry is repointed;
 * *cow_src / *cow_dst then name the block to copy before writing (else both
 * are -1).  *slot_out receives the slot.  PKV_ENOMEM if no block is free (the
 * table is unchanged), PKV_EINVAL on inconsistent arguments.
 */
pkv_status pkv_pool_append(pkv_pool* pool, int32_t* table, int32_t table_capacity,
                           int32_t* table_len, int32_t seq_len, int block_size,
                           int32_t* slot_out, int32_t* cow_src, int32_t* cow_dst);

/* Pool occupancy: free blocks, blocks in use, blocks with count > 1. */
pkv_status pkv_pool_stats(const pkv_pool* pool, int32_t* free_blocks, int32_t* used_blocks,
                          int32_t* shared_blocks);
/* Copies the free list, front first, into out[0 .. min(n, cap)); *n = its length. */
pkv_status pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n);

/* ------------------------------------------------------------------------ */
/* Host block reuse                                                          */
/* ------------------------------------------------------------------------ */
/*
 * Prefix cache ([P2] s.11 "Prefix reuse"): a completed block is stored
 * under its full token prefix (kept as a chain of (parent entry, the
 * block's own block_size tokens), compared in full: no false match), so a
 * request starting with the same tokens reuses it.  The cache holds one
 * reference (pkv_pool_incref) per cached block.  Host only; tokens are
 * int32 ids.
 */
typedef struct pkv_prefix_cache pkv_prefix_cache;

/* A cache over `pool` (not owned; it must outlive the cache).  NULL on error. */
pkv_prefix_cache* pkv_prefix_cache_create(pkv_pool* pool, int block_size);
/* Releases the cache's references and frees it. */
void pkv_prefix_cache_destroy(pkv_prefix_cache* cache);

/*
 * The leading full blocks of tokens[0 .. n_tokens) that are cached, up to
 * the first miss and at most max_blocks: their physical blocks go to
 * blocks_out[0 .. *n_matched), and the caller receives one pool reference
 * for each (release with pkv_pool_decref when the sequence ends).
 */
pkv_status pkv_prefix_cache_match(pkv_prefix_cache* cache, const int32_t* tokens, int n_tokens,
                                  int32_t* blocks_out, int max_blocks, int* n_matched);

/*
 * Stores the full blocks of tokens[0 .. n_tokens) held in blocks[0 ..
 * n_blocks) (a sequence's table); a block whose prefix is already cached
 * keeps the cached entry.  The cache takes a reference to each block it
 * adds; *n_added (may be NULL) receives their number.
 */
pkv_status pkv_prefix_cache_insert(pkv_prefix_cache* cache, const int32_t* tokens, int n_tokens,
                                   const int32_t* blocks, int n_blocks, int* n_added);

/*
 * Drops up to n_wanted entries, least recently used first, among those with
 * no cached entry after them and whose block only the cache holds; their
 * blocks go back to the pool's free list.  *n_evicted (may be NULL)
 * receives the count.
 */
pkv_status pkv_prefix_cache_evict(pkv_prefix_cache* cache, int n_wanted, int* n_evicted);

/* Entries in the cache (-1 for NULL). */
int pkv_prefix_cache_size(const pkv_prefix_cache* cache);

/*
 * H2O retention ([P2] s.9 "Eviction"): of n positions with accumulated
 * attention scores, keep the latest min(recent_count, budget) and give the
 * rest of the budget to the older positions with the largest scores
 * (earlier position first among equal scores).  kept_out[0 .. *n_kept)
 * receives the kept positions in increasing order (all n when budget >= n).
 * NaN scores give PKV_EINVAL.
 */
pkv_status pkv_h2o_retain(const float* scores, int n, int budget, int recent_count, int32_t* kept_out,
                          int* n_kept);

/* ------------------------------------------------------------------------
 * Measurement
 * ------------------------------------------------------------------------ */

/*
 * Streaming-read probe: reads `bytes` bytes from device memory at src once
 * (16-byte non-temporal loads, every CU busy) and stores one 32-bit fold of
 * the data per workgroup into sink (device, at least
 * pkv_stream_read_sink_words() words), so that nothing is skipped.  Timed
 * around it, it gives the box's streaming-read ceiling that the decode's
 * HBM figures are set against.  bytes must be a multiple of 16 and src
 * 16-byte aligned.
 */
int pkv_stream_read_sink_words(void);
pkv_status pkv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
