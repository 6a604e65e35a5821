// Internal declarations shared by the host-side translation units.
#ifndef PKV_INTERNAL_H_
#define PKV_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Records the thread-local error message and returns `st`.
pkv_status fail(pkv_status st, const char* fmt, ...);
void set_error(const char* fmt, ...);
void clear_error();

inline int dtype_bytes(int dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_BF16:
    case PKV_F16: return 2;
    case PKV_I8:
    case PKV_FP8E4M3:
    case PKV_FP8E5M2:
    case PKV_I4: return 1;   // INT4: a byte holds two elements (see row_bytes)
    default: return 0;
  }
}

inline bool is_float_storage(int dt) { return dt == PKV_F32 || dt == PKV_BF16 || dt == PKV_F16; }
inline bool is_code_storage(int dt) {
  return dt == PKV_I8 || dt == PKV_FP8E4M3 || dt == PKV_FP8E5M2 || dt == PKV_I4;
}
// Bytes of one cache row (one token, one KV head) of head_dim elements.
inline int row_bytes(int dt, int head_dim) { return dt == PKV_I4 ? head_dim / 2 : head_dim * dtype_bytes(dt); }

// Decode-attention launch description shared by the partition and merge passes.
struct AttnArgs {
  void* out;
  const void* query;
  int q_dtype;
  const void* k_cache;
  const void* v_cache;
  int kv_dtype;
  const float* k_scales;
  const float* v_scales;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* seq_lens;
  int num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks;
  float sm_scale;
  int partition_size;  // resolved (never 0)
  int num_partitions;  // per sequence, from max_blocks_per_seq * block_size
  // 16-bit / code caches: workgroups along the sequence axis, blocks a
  // workgroup's list holds, fewest partitions per workgroup, and whether a
  // sequence can be cut over several workgroups (merge needed)
  int num_slots, list_cap, min_units;
  bool may_split;
  unsigned flags;  // PKV_DECODE_* bits
  int sink_tokens, window_tokens;
  // Partial results.  A record holds acc[G][D] (unnormalised fp32
  // accumulators of the group's query heads), then m[16] and l[16] (running
  // max in the log2 domain and softmax denominator; entries >= G unused).
  // 16-bit / code caches: two record slots per (workgroup, KV head); fp32
  // caches: one record per (sequence, KV head, partition), partition fastest.
  float* ws;
  int* plan;   // wave path: [num_seqs][4] ints for the merge, before the records
  // selected decode: [S][Hkv][budget] (physical block, logical block) pairs
  // in logical order; the units are these pages (partition_size 16)
  const int32_t* selected;
  int budget;
  int qtok;    // query tokens per sequence (0 or 1: one)
  // grouped scales: K channel scales [NB][Hkv][D] (k_scales then holds each
  // tile's largest channel scale) and v_scales per token [NB][Hkv][16]
  const float* k_chan;
  // fused slot write of each sequence's new token (16-bit caches)
  const void* new_k;
  const void* new_v;
  const int32_t* positions;
  int32_t* slots_out;
  // shared-prefix decode: block_tables points at entry prefix_blocks of row
  // 0, rows are table_stride entries apart (0: max_blocks_per_seq) and
  // lengths count from token len_off; prefix holds one record per
  // (sequence, query head) of the shared blocks (prefix_record_floats);
  // srec one partial record per (sequence, KV head) for sequences the
  // decode finishes in one piece (their output is written by the merge,
  // which then runs for every sequence and needs the plan area)
  int table_stride;
  int len_off;
  const float* prefix;
  float* srec;
  void* stream;
};

// Floats in one partial record for group size G and head_dim D.
inline size_t partial_record_floats(int G, int D) { return (size_t)G * D + 32; }
inline size_t whole_record_area_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int D) {
  return ((size_t)num_seqs * num_kv_heads * partial_record_floats(num_q_heads / num_kv_heads, D) * 4 + 255) &
         ~(size_t)255;
}

// Floats in one shared-prefix record: acc[D] (unnormalised), m (log2
// domain), l, two unused.
inline size_t prefix_record_floats(int D) { return (size_t)D + 4; }
// Bytes of the shared-prefix records of a batch (256-byte aligned).
inline size_t prefix_area_bytes(int num_seqs, int num_q_heads, int D) {
  return ((size_t)num_seqs * num_q_heads * prefix_record_floats(D) * 4 + 255) & ~(size_t)255;
}
// Bytes of the shared-prefix decode's per-(sequence, KV head) records of
// whole sequences (256-byte aligned); defined after partial_record_floats.
inline size_t whole_record_area_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int D);

// KV heads (one wave each) per workgroup of the 16-bit / code-cache decode.
inline int wave_group_size(int num_kv_heads) { return num_kv_heads < 8 ? num_kv_heads : 8; }
// Blocks a workgroup of that decode takes at most (its block list in LDS).
inline int decode_list_cap(int num_kv_heads) { return 128 * wave_group_size(num_kv_heads); }
// Workgroups along the sequence axis of that decode: enough to fill every
// compute unit at two waves per SIMD, at least one per sequence, and enough
// that no workgroup's share of the partitions exceeds its block list.
// cus: compute units the decode runs on (0: all of the device's)
int decode_slots(int num_seqs, int num_kv_heads, int num_partitions, int partition_size, int cus = 0);
int device_cu_count();
// Bytes at the start of the wave path's workspace that hold, per sequence,
// the slot of its first partial record and the first and last workgroups it
// reaches (four int32), written by the decode for the merge; the records
// follow.
inline size_t plan_area_bytes(int num_seqs) { return ((size_t)num_seqs * 16 + 255) & ~(size_t)255; }
// Fewest partitions a workgroup takes: enough for 80 tokens (5 blocks), so
// that its fixed costs stay small next to its stream, while small batches
// still spread over many compute units (a 4 + 4092 StreamingLLM window over
// four sequences keeps 207 workgroups busy, against 129 at 8 blocks).
inline int min_units_per_wave(int partition_size) {
  const int m = 80 / partition_size;
  return m < 1 ? 1 : m;
}
// Bytes of workspace the split decode needs for a cache of kv_dtype: fp32
// records per (sequence, KV head, partition) for fp32 caches; the plan area
// and two records per (workgroup, KV head) otherwise; 0 if no sequence can
// be split.
size_t workspace_total(int kv_dtype, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int num_partitions, int partition_size);

// Kernel launchers (defined in the .hip files).  They assume validated
// arguments and return a hipError_t cast to int.
int launch_paged_attn_partition(const AttnArgs& a);
int launch_paged_attn_merge(const AttnArgs& a);
// Several query tokens per sequence with more than 16 query rows per KV head
// (a chunk of prefill): the query-tile pass, written straight to `out`.
int launch_chunk_attn(const AttnArgs& a);
// Shared-prefix pass: one record per (sequence, query head) of attention
// over the prefix_blocks blocks listed at `table`.
int launch_prefix_attn(const void* query, int q_dtype, const void* k_cache, const void* v_cache,
                       const int32_t* table, int prefix_blocks, float* records, int num_seqs, int num_q_heads,
                       int num_kv_heads, int head_dim, int num_blocks, float sm_scale, void* stream);
int launch_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* seq_ids, const int32_t* positions, int num_tokens,
                        int num_seqs, int block_size, int num_blocks, void* stream);
int launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                             int elem_bytes, const int32_t* slot_mapping, int num_tokens,
                             int num_blocks, int block_size, int num_kv_heads, int head_dim,
                             void* stream);
int launch_append_kv(const void* key, const void* value, void* k_cache, void* v_cache, int elem_bytes,
                     const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_ids,
                     const int32_t* positions, int32_t* slot_mapping, int num_tokens, int num_seqs,
                     int num_blocks, int block_size, int num_kv_heads, int head_dim, void* stream);
int launch_copy_blocks(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                       const int32_t* src_dst, int n, int elem_bytes, int num_blocks, int block_size,
                       int num_kv_heads, int head_dim, void* stream);
int launch_append_quantized(const void* key, const void* value, int src_dtype, void* k_tail, void* v_tail,
                            void* k_codes, void* v_codes, int code_dtype, float* k_scales, float* v_scales,
                            float* k_group, float* v_group, const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* positions, int num_seqs, int num_blocks, int num_kv_heads, int head_dim,
                            void* stream);
// Shared-prefix decode: (32-row tile, KV head) items of the prefix pass,
// and the prefix workgroups of a combined launch on a device of `cus`
// compute units (0: launch the prefix pass on its own).
int prefix_item_count(int num_seqs, int num_q_heads, int num_kv_heads);
int prefix_workgroups(int num_seqs, int num_q_heads, int num_kv_heads, int cus);
// The combined launch: the decode past the prefix (a.num_slots slots), then
// pfx_wgs workgroups along x of prefix items.
int launch_shared_prefix_decode(const AttnArgs& a, const int32_t* prefix_table, int prefix_blocks, float* prefix_rec,
                                int pfx_wgs);
int launch_quest_summarize(const void* k_cache, int kv_dtype, void* k_summary, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_blocks,
                           int num_kv_heads, int head_dim, int last_only, void* stream);
int launch_quest_select(const void* query, int q_dtype, const void* k_summary, const int32_t* block_tables,
                        int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_dim, int num_blocks, int budget, int32_t* selected,
                        void* scratch, void* stream);
// streaming-read probe: workgroups (4 per CU) and their launcher
constexpr int kStreamReadBlocks = 1024;
int launch_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);
int launch_quantize_kv_grouped(const void* src_cache, int src_dtype, void* dst_codes, int code_dtype,
                               float* tile_scales, float* group_scales, int group, const int32_t* block_ids,
                               int n_blocks, int num_blocks, int num_kv_heads, int head_dim, void* stream);
int launch_quantize_kv(const void* src_cache, int src_dtype, void* dst_codes, int code_dtype,
                       float* dst_scales, const int32_t* block_ids, int n_blocks, int num_blocks,
                       int block_size, int num_kv_heads, int head_dim, void* stream);

}  // namespace pkv

#endif  // PKV_INTERNAL_H_
