// The C ABI: argument validation, partition choice, workspace layout and
// kernel dispatch on the caller's stream.  Host code only.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {

static pkv_status hip_status(int err, const char* where) {
  if (err == hipSuccess) return PKV_OK;
  return fail(PKV_EHIP, "%s: %s", where, hipGetErrorString((hipError_t)err));
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Compute units of the current device (256 when none can be queried, e.g.
// on a host without a GPU, so that sizes computed there match MI355X).
int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cache[dev] = n;
  }
  return cache[dev];
}

int decode_slots(int num_seqs, int num_kv_heads, int num_partitions, int partition_size, int cus) {
  constexpr int kWavesPerCU = 8;   // two waves per SIMD: the wave kernel's register budget
  if (cus <= 0) cus = device_cu_count();
  long long k = ((long long)kWavesPerCU * cus + num_kv_heads - 1) / num_kv_heads;
  if (k < num_seqs) k = num_seqs;
  // a workgroup takes at most ceil(units / k) partitions (or the minimum),
  // or, when the split balances blocks, its share of the blocks plus up to
  // one partition less a block: both must fit its block list
  const long long blocks_per_unit = partition_size / 16 > 0 ? partition_size / 16 : 1;
  const long long cap = decode_list_cap(num_kv_heads);
  // (the decode balances blocks only when 3 blocks_per_unit <= cap)
  const long long units_cap = 3 * blocks_per_unit <= cap ? (cap - blocks_per_unit + 1) / blocks_per_unit
                                                         : cap / blocks_per_unit;
  if (units_cap > 0) {
    const long long need = ((long long)num_seqs * num_partitions + units_cap - 1) / units_cap;
    if (k < need) k = need;
  }
  return k > 0x7FFFFFFF ? 0x7FFFFFFF : (int)k;
}

size_t workspace_total(int kv_dtype, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int num_partitions, int partition_size) {
  if (num_partitions <= 1 || num_seqs <= 0) return 0;
  const int G = num_q_heads / num_kv_heads;
  const size_t rec = partial_record_floats(G, head_dim) * sizeof(float);
  if (kv_dtype == PKV_F32) return align256((size_t)num_seqs * num_kv_heads * num_partitions * rec);
  const size_t slots = 2 * (size_t)decode_slots(num_seqs, num_kv_heads, num_partitions, partition_size);
  return align256(plan_area_bytes(num_seqs) + slots * num_kv_heads * rec);
}

static bool check_env() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("PKV_CHECK");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

// Resolve a user partition size (0 = auto) for the given shape.
static int resolve_partition(int kv_dtype, int max_len, int block_size, int psize) {
  if (psize > 0) return psize;
  // Bounds up to 512 tokens run as one pass without partials.  Longer ones
  // are split at block granularity for the 16-bit and code caches, whose
  // decode balances its workgroups to the block, and at 64 tokens for fp32.
  const int single = ((max_len + block_size - 1) / block_size) * block_size;
  if (max_len <= 512) return single > 0 ? single : block_size;
  return kv_dtype == PKV_F32 ? 64 : block_size;
}

}  // namespace pkv

using namespace pkv;


extern "C" int pkv_stream_read_sink_words(void) { return kStreamReadBlocks; }

extern "C" pkv_status pkv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes % 16) return fail(PKV_EINVAL, "pkv_stream_read: bytes must be a multiple of 16");
  if (bytes == 0) return PKV_OK;
  if (!src || !sink) return fail(PKV_EINVAL, "pkv_stream_read: null pointer");
  if (((uintptr_t)src) & 15) return fail(PKV_EINVAL, "pkv_stream_read: src must be 16-byte aligned");
  return hip_status(launch_stream_read(src, bytes, sink, stream), "pkv_stream_read");
}

extern "C" int pkv_paged_attn_partition_size(int kv_dtype, int max_seq_len, int block_size) {
  if (block_size <= 0 || max_seq_len < 0) return 0;
  return resolve_partition(kv_dtype, max_seq_len, block_size, 0);
}

extern "C" int pkv_paged_attn_num_partitions(int kv_dtype, int max_seq_len, int block_size, int partition_size) {
  if (block_size <= 0 || max_seq_len < 0 || partition_size < 0) return 0;
  if (partition_size > 0 && partition_size % block_size) return 0;
  const int ps = resolve_partition(kv_dtype, max_seq_len, block_size, partition_size);
  const int n = (max_seq_len + ps - 1) / ps;
  return n < 1 ? 1 : n;
}

extern "C" size_t pkv_paged_attn_workspace_bytes(int kv_dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                                                 int head_dim, int max_seq_len, int partition_size) {
  const int np = pkv_paged_attn_num_partitions(kv_dtype, max_seq_len, 16, partition_size);
  if (np <= 1 || num_seqs <= 0) return 0;
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads) return 0;
  const int ps = resolve_partition(kv_dtype, max_seq_len, 16, partition_size);
  return workspace_total(kv_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, np, ps);
}

// Device arrays -> host, then pkv_validate_tables (PKV_CHECK=1 only).
static pkv_status device_check(const int32_t* block_tables, int mbs, const int32_t* seq_lens, int num_seqs,
                               int block_size, int num_blocks, const int32_t* slots, int num_tokens,
                               void* stream) {
  std::vector<int32_t> bt((size_t)num_seqs * mbs), sl(num_seqs), sm(slots ? num_tokens : 0);
  hipStream_t st = (hipStream_t)stream;
  int e = hipSuccess;
  if (num_seqs > 0 && block_tables)
    e |= hipMemcpyAsync(bt.data(), block_tables, bt.size() * 4, hipMemcpyDeviceToHost, st);
  if (num_seqs > 0 && seq_lens) e |= hipMemcpyAsync(sl.data(), seq_lens, sl.size() * 4, hipMemcpyDeviceToHost, st);
  if (slots && num_tokens > 0) e |= hipMemcpyAsync(sm.data(), slots, sm.size() * 4, hipMemcpyDeviceToHost, st);
  e |= hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PKV_EHIP, "PKV_CHECK: copying tables to the host failed");
  return pkv_validate_tables(block_tables ? bt.data() : nullptr, mbs, seq_lens ? sl.data() : nullptr,
                             seq_lens ? num_seqs : 0, block_size, num_blocks, slots ? sm.data() : nullptr,
                             num_tokens);
}

static pkv_status check_cache_shape(const char* who, int block_size, int num_kv_heads, int head_dim) {
  if (block_size != 16) return fail(PKV_EUNSUPPORTED, "%s: block_size must be 16", who);
  if (num_kv_heads <= 0) return fail(PKV_EINVAL, "%s: num_kv_heads must be positive", who);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim must be 64 or 128", who);
  return PKV_OK;
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------
static pkv_status prepare_attn(AttnArgs& a, const char* who, void* workspace, size_t workspace_bytes,
                               bool need_inputs) {
  if (a.num_seqs < 0 || a.num_q_heads <= 0 || a.num_kv_heads <= 0 || a.max_blocks_per_seq < 0 || a.num_blocks < 0)
    return fail(PKV_EINVAL, "%s: negative or zero size", who);
  if (a.num_q_heads % a.num_kv_heads)
    return fail(PKV_EINVAL, "%s: num_q_heads %% num_kv_heads != 0", who);
  if (a.qtok < 1) a.qtok = 1;
  if (a.num_q_heads / a.num_kv_heads > 16)
    return fail(PKV_EUNSUPPORTED, "%s: query group size above 16 is not built", who);
  if (a.qtok > 1) {
    if ((long long)(a.num_q_heads / a.num_kv_heads) * a.qtok > 16)
      return fail(PKV_EUNSUPPORTED, "%s: query tokens x group size above 16 is not built", who);
    if (a.q_dtype == PKV_F32) return fail(PKV_EUNSUPPORTED, "%s: several query tokens need a 16-bit query", who);
    if (a.sink_tokens || a.window_tokens || a.selected)
      return fail(PKV_EUNSUPPORTED, "%s: several query tokens take neither a keep-mask nor a selection", who);
  }
  if (a.head_dim != 64 && a.head_dim != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim must be 64 or 128", who);
  if (a.block_size != 16) return fail(PKV_EUNSUPPORTED, "%s: block_size must be 16", who);
  if (a.q_dtype != PKV_F32 && a.q_dtype != PKV_BF16 && a.q_dtype != PKV_F16)
    return fail(PKV_EUNSUPPORTED, "%s: query dtype must be f32, bf16 or f16", who);
  if (need_inputs) {
    const bool same = a.kv_dtype == a.q_dtype;
    const bool codes = is_code_storage(a.kv_dtype) && (a.q_dtype == PKV_BF16 || a.q_dtype == PKV_F16);
    if (!same && !codes)
      return fail(PKV_EUNSUPPORTED, "%s: kv dtype must equal the query dtype, or be a code type with a 16-bit query",
                  who);
    if (codes && (!a.k_scales || !a.v_scales)) return fail(PKV_EINVAL, "%s: quantised cache needs k/v scales", who);
    if (a.kv_dtype == PKV_I4 && a.head_dim != 128)
      return fail(PKV_EUNSUPPORTED, "%s: INT4 caches are built for head_dim 128", who);
    if (a.sink_tokens < 0 || a.window_tokens < 0) return fail(PKV_EINVAL, "%s: negative sink/window", who);
    if (a.flags & ~(unsigned)PKV_DECODE_STREAM_KV) return fail(PKV_EINVAL, "%s: unknown flags 0x%x", who, a.flags);
  }
  if (a.partition_size < 0 || (a.partition_size > 0 && a.partition_size % a.block_size))
    return fail(PKV_EINVAL, "%s: partition_size must be 0 or a positive multiple of block_size", who);
  const int max_len = a.max_blocks_per_seq * a.block_size;
  a.partition_size = resolve_partition(a.kv_dtype, max_len, a.block_size, a.partition_size);
  a.num_partitions = (max_len + a.partition_size - 1) / a.partition_size;
  if (a.num_partitions < 1) a.num_partitions = 1;
  if (a.num_seqs == 0) return PKV_OK;
  if (!a.out || !a.seq_lens) return fail(PKV_EINVAL, "%s: null pointer argument", who);
  if (need_inputs && (!a.query || !a.k_cache || !a.v_cache || (!a.block_tables && !a.selected)))
    return fail(PKV_EINVAL, "%s: null pointer argument", who);
  const bool wave_path = a.q_dtype != PKV_F32;
  if (wave_path) {
    // the decode keeps sequence numbers in 23 bits, table offsets and unit
    // counts in 31
    if (a.num_seqs >= (1 << 23) || (long long)a.num_seqs * a.max_blocks_per_seq >= (1LL << 29) ||
        (long long)a.num_seqs * a.num_partitions >= (1LL << 30))
      return fail(PKV_EUNSUPPORTED, "%s: batch too large (num_seqs * max_blocks_per_seq >= 2^29)", who);
    // block offsets are formed as num_blocks * num_kv_heads * 4 in 31 bits
    if ((long long)a.num_blocks * a.num_kv_heads >= (1LL << 29))
      return fail(PKV_EUNSUPPORTED, "%s: pool too large (num_blocks * num_kv_heads >= 2^29)", who);
    a.list_cap = decode_list_cap(a.num_kv_heads);
    if (a.partition_size / a.block_size > a.list_cap)
      return fail(PKV_EINVAL, "%s: partition_size above %d tokens", who, a.list_cap * a.block_size);
    a.num_slots = decode_slots(a.num_seqs, a.num_kv_heads, a.num_partitions, a.partition_size);
    a.min_units = min_units_per_wave(a.partition_size);
  }
  a.may_split = a.num_partitions > 1;
  a.ws = nullptr;
  a.plan = nullptr;
  // the shared-prefix decode merges every sequence: it needs the plan area
  // even when no sequence can be cut
  if (a.may_split || (a.srec && wave_path)) {
    // records hold one row per (query token, query head) of a group
    const size_t total = a.may_split ? workspace_total(a.kv_dtype, a.num_seqs, a.num_q_heads * a.qtok,
                                                       a.num_kv_heads, a.head_dim, a.num_partitions,
                                                       a.partition_size)
                                     : plan_area_bytes(a.num_seqs);
    if (!workspace || workspace_bytes < total)
      return fail(PKV_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, total, workspace_bytes);
    if (((uintptr_t)workspace) & 127) return fail(PKV_EINVAL, "%s: workspace must be 128-byte aligned", who);
    if (!wave_path) {
      a.ws = (float*)workspace;
    } else {
      a.plan = (int*)workspace;
      a.ws = a.may_split ? (float*)((char*)workspace + plan_area_bytes(a.num_seqs)) : nullptr;
    }
  }
  return PKV_OK;
}

#define PKV_ATTN_ARGS                                                                                        \
  void *out, const void *query, int q_dtype, const void *k_cache, const void *v_cache, int kv_dtype,          \
      const float *k_scales, const float *v_scales, const int32_t *block_tables, int max_blocks_per_seq,      \
      const int32_t *seq_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size, \
      int num_blocks, float sm_scale, int partition_size, int sink_tokens, int window_tokens, unsigned flags,  \
      void *workspace, size_t workspace_bytes, void *stream

static AttnArgs fill_args(void* out, const void* query, int q_dtype, const void* k_cache, const void* v_cache,
                          int kv_dtype, const float* k_scales, const float* v_scales, const int32_t* block_tables,
                          int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_q_heads,
                          int num_kv_heads, int head_dim, int block_size, int num_blocks, float sm_scale,
                          int partition_size, int sink_tokens, int window_tokens, unsigned flags,
                          void* stream) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.out = out;
  a.query = query;
  a.q_dtype = q_dtype;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_dtype = kv_dtype;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.sm_scale = sm_scale;
  a.partition_size = partition_size;
  a.sink_tokens = sink_tokens;
  a.window_tokens = window_tokens;
  a.flags = flags;
  a.stream = stream;
  return a;
}

static pkv_status run_attn(bool do_partition, bool do_merge, PKV_ATTN_ARGS) {
  AttnArgs a = fill_args(out, query, q_dtype, k_cache, v_cache, kv_dtype, k_scales, v_scales, block_tables,
                         max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         num_blocks, sm_scale, partition_size, sink_tokens, window_tokens, flags, stream);
  const char* who = do_partition ? (do_merge ? "pkv_paged_attn_decode" : "pkv_paged_attn_partition")
                                 : "pkv_paged_attn_merge";
  pkv_status st = prepare_attn(a, who, workspace, workspace_bytes, do_partition);
  if (st != PKV_OK || num_seqs == 0) return st;
  if (do_partition && check_env()) {
    st = device_check(block_tables, max_blocks_per_seq, seq_lens, num_seqs, block_size, num_blocks, nullptr, 0,
                      stream);
    if (st != PKV_OK) return st;
  }
  if (do_partition) {
    st = hip_status(launch_paged_attn_partition(a), who);
    if (st != PKV_OK) return st;
  }
  if (do_merge) st = hip_status(launch_paged_attn_merge(a), who);
  return st;
}

extern "C" pkv_status pkv_paged_attn_decode(PKV_ATTN_ARGS) {
  return run_attn(true, true, out, query, q_dtype, k_cache, v_cache, kv_dtype, k_scales, v_scales, block_tables,
                  max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                  num_blocks, sm_scale, partition_size, sink_tokens, window_tokens, flags, workspace,
                  workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// decode without a caller workspace: the scratch is a fixed device array
// ---------------------------------------------------------------------------
namespace pkv {

// The decode's scratch (merge plan and partial records) for callers that
// cannot allocate.  Every GPU the library runs on holds its own copy of this
// array until the process ends.  Host code must never pass `scratch` itself to
// a kernel: on the host the name stands for a host-side shadow, not the device
// copy.  Its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];   // device address of `scratch`, per device

static pkv_status scratch_address(void** out, const char* who) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PKV_EHIP, "%s: hipGetDevice failed", who);
  if (dev < 0 || dev >= 64) return fail(PKV_EUNSUPPORTED, "%s: device %d above 63", who, dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PKV_EHIP, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace pkv

extern "C" size_t pkv_paged_attn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" pkv_status pkv_paged_attn_decode_noalloc(
    void* out, const void* query, int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
    const float* k_scales, const float* v_scales, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* seq_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int num_blocks, float sm_scale, int partition_size, int sink_tokens, int window_tokens, unsigned flags,
    void* stream) {
  const char* who = "pkv_paged_attn_decode_noalloc";
  AttnArgs a = fill_args(out, query, q_dtype, k_cache, v_cache, kv_dtype, k_scales, v_scales, block_tables,
                         max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         num_blocks, sm_scale, partition_size, sink_tokens, window_tokens, flags, stream);
  // the same size rule as pkv_paged_attn_workspace_bytes, checked against
  // the fixed array before anything is launched
  if (num_seqs > 0 && num_kv_heads > 0 && num_q_heads > 0 && num_q_heads % num_kv_heads == 0 &&
      max_blocks_per_seq >= 0 && block_size == 16 && partition_size >= 0) {
    const size_t need = pkv_paged_attn_workspace_bytes(kv_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                       max_blocks_per_seq * block_size, partition_size);
    if (need > kNoAllocScratchBytes)
      return fail(PKV_EWORKSPACE, "%s: the decode needs %zu bytes of scratch, above the fixed %zu", who, need,
                  kNoAllocScratchBytes);
  }
  void* ws = nullptr;
  if (num_seqs > 0) {
    const pkv_status st = scratch_address(&ws, who);
    if (st != PKV_OK) return st;
  }
  pkv_status st = prepare_attn(a, who, ws, kNoAllocScratchBytes, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  st = hip_status(launch_paged_attn_partition(a), who);
  if (st != PKV_OK) return st;
  return hip_status(launch_paged_attn_merge(a), who);
}

extern "C" pkv_status pkv_paged_attn_partition(PKV_ATTN_ARGS) {
  return run_attn(true, false, out, query, q_dtype, k_cache, v_cache, kv_dtype, k_scales, v_scales,
                  block_tables, max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                  block_size, num_blocks, sm_scale, partition_size, sink_tokens, window_tokens, flags, workspace,
                  workspace_bytes, stream);
}

extern "C" pkv_status pkv_paged_attn_decode_multi(
    void* out, const void* query, int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
    const float* k_scales, const float* v_scales, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* seq_lens, int num_seqs, int num_query_tokens, int num_q_heads, int num_kv_heads, int head_dim,
    int block_size, int num_blocks, float sm_scale, int partition_size, unsigned flags, void* workspace,
    size_t workspace_bytes, void* stream) {
  const char* who = "pkv_paged_attn_decode_multi";
  if (num_query_tokens < 1) return fail(PKV_EINVAL, "%s: num_query_tokens must be positive", who);
  AttnArgs a = fill_args(out, query, q_dtype, k_cache, v_cache, kv_dtype, k_scales, v_scales, block_tables,
                         max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         num_blocks, sm_scale, partition_size, 0, 0, flags, stream);
  a.qtok = num_query_tokens;
  if (num_kv_heads > 0 && num_q_heads > 0 && num_q_heads % num_kv_heads == 0 &&
      (long long)(num_q_heads / num_kv_heads) * num_query_tokens > 16) {
    // more query rows per KV head than the decode's 16 MFMA columns: the
    // query-tile pass (a chunk of prefill), which needs no workspace
    if (num_seqs < 0 || max_blocks_per_seq < 0 || num_blocks < 0) return fail(PKV_EINVAL, "%s: negative size", who);
    if (q_dtype != PKV_BF16 && q_dtype != PKV_F16)
      return fail(PKV_EUNSUPPORTED, "%s: more than 16 query rows per KV head need a bf16 or f16 query", who);
    if (kv_dtype != q_dtype)
      return fail(PKV_EUNSUPPORTED, "%s: more than 16 query rows per KV head are built for 16-bit caches", who);
    pkv_status st = check_cache_shape(who, block_size, num_kv_heads, head_dim);
    if (st != PKV_OK) return st;
    if (partition_size < 0 || (partition_size > 0 && partition_size % block_size))
      return fail(PKV_EINVAL, "%s: partition_size must be 0 or a positive multiple of block_size", who);
    if (flags & ~(unsigned)PKV_DECODE_STREAM_KV) return fail(PKV_EINVAL, "%s: unknown flags 0x%x", who, flags);
    // one workgroup per 32 query rows of each (sequence, KV head), the pairs
    // padded to a multiple of 8
    const long long tiles = ((long long)num_query_tokens * (num_q_heads / num_kv_heads) + 31) / 32;
    if (((long long)num_seqs * num_kv_heads + 7) / 8 * 8 * tiles >= (1LL << 31))
      return fail(PKV_EUNSUPPORTED, "%s: grid too large (2^31 workgroups or more)", who);
    if (num_seqs == 0) return PKV_OK;
    if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens)
      return fail(PKV_EINVAL, "%s: null pointer argument", who);
    return hip_status(launch_chunk_attn(a), who);
  }
  pkv_status st = prepare_attn(a, who, workspace, workspace_bytes, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  st = hip_status(launch_paged_attn_partition(a), who);
  if (st != PKV_OK) return st;
  return hip_status(launch_paged_attn_merge(a), who);
}

extern "C" pkv_status pkv_paged_attn_decode_selected(
    void* out, const void* query, int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
    const float* k_scales, const float* v_scales, const int32_t* selected, int budget_blocks,
    const int32_t* seq_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int num_blocks, float sm_scale, unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "pkv_paged_attn_decode_selected";
  if (budget_blocks <= 0) return fail(PKV_EINVAL, "%s: budget_blocks must be positive", who);
  if (q_dtype == PKV_F32) return fail(PKV_EUNSUPPORTED, "%s: fp32 caches are not built for selected reads", who);
  if (num_seqs > 0 && num_kv_heads > 0 &&
      (long long)num_seqs * num_kv_heads * budget_blocks * 8 >= (1LL << 31))
    return fail(PKV_EUNSUPPORTED, "%s: selection of 2^31 bytes or more", who);
  // the selection's pages are the units: one-block partitions over a bound
  // of budget_blocks blocks
  AttnArgs a = fill_args(out, query, q_dtype, k_cache, v_cache, kv_dtype, k_scales, v_scales, nullptr, budget_blocks,
                         seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, sm_scale,
                         16, 0, 0, flags, stream);
  a.selected = selected;
  a.budget = budget_blocks;
  if (num_seqs > 0 && !selected) return fail(PKV_EINVAL, "%s: null pointer argument", who);
  pkv_status st = prepare_attn(a, who, workspace, workspace_bytes, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  st = hip_status(launch_paged_attn_partition(a), who);
  if (st != PKV_OK) return st;
  return hip_status(launch_paged_attn_merge(a), who);
}

extern "C" pkv_status pkv_paged_attn_decode_append(
    void* out, const void* query, int q_dtype, void* k_cache, void* v_cache, int kv_dtype, const void* key,
    const void* value, const int32_t* positions, int32_t* slot_mapping_out, const int32_t* block_tables,
    int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int block_size, int num_blocks, float sm_scale, int partition_size, int sink_tokens, int window_tokens,
    unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "pkv_paged_attn_decode_append";
  if (kv_dtype != q_dtype || (kv_dtype != PKV_BF16 && kv_dtype != PKV_F16))
    return fail(PKV_EUNSUPPORTED, "%s: the fused write is built for bf16 / f16 caches of the query dtype", who);
  if (num_seqs > 0 && (!key || !value || !positions)) return fail(PKV_EINVAL, "%s: null pointer argument", who);
  AttnArgs a = fill_args(out, query, q_dtype, k_cache, v_cache, kv_dtype, nullptr, nullptr, block_tables,
                         max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         num_blocks, sm_scale, partition_size, sink_tokens, window_tokens, flags, stream);
  a.new_k = key;
  a.new_v = value;
  a.positions = positions;
  a.slots_out = slot_mapping_out;
  pkv_status st = prepare_attn(a, who, workspace, workspace_bytes, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  if (check_env()) {
    st = device_check(block_tables, max_blocks_per_seq, seq_lens, num_seqs, block_size, num_blocks, nullptr, 0,
                      stream);
    if (st != PKV_OK) return st;
  }
  st = hip_status(launch_paged_attn_partition(a), who);
  if (st != PKV_OK) return st;
  return hip_status(launch_paged_attn_merge(a), who);
}

extern "C" pkv_status pkv_paged_attn_decode_grouped(
    void* out, const void* query, int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
    const float* k_tile_scales, const float* k_channel_scales, const float* v_token_scales,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_q_heads,
    int num_kv_heads, int head_dim, int block_size, int num_blocks, float sm_scale, int partition_size,
    unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "pkv_paged_attn_decode_grouped";
  if (kv_dtype != PKV_I8 && kv_dtype != PKV_I4)
    return fail(PKV_EUNSUPPORTED, "%s: grouped scales are built for i8 and i4 codes", who);
  if (q_dtype != PKV_BF16 && q_dtype != PKV_F16) return fail(PKV_EUNSUPPORTED, "%s: query must be bf16 or f16", who);
  if (num_seqs > 0 && (!k_tile_scales || !k_channel_scales || !v_token_scales))
    return fail(PKV_EINVAL, "%s: null scale pointer", who);
  // token scales are addressed as num_blocks * num_kv_heads * 64 bytes in 31 bits
  if ((long long)num_blocks * num_kv_heads >= (1LL << 25))
    return fail(PKV_EUNSUPPORTED, "%s: pool too large (num_blocks * num_kv_heads >= 2^25)", who);
  AttnArgs a = fill_args(out, query, q_dtype, k_cache, v_cache, kv_dtype, k_tile_scales, v_token_scales,
                         block_tables, max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                         block_size, num_blocks, sm_scale, partition_size, 0, 0, flags, stream);
  a.k_chan = k_channel_scales;
  pkv_status st = prepare_attn(a, who, workspace, workspace_bytes, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  if (check_env()) {
    st = device_check(block_tables, max_blocks_per_seq, seq_lens, num_seqs, block_size, num_blocks, nullptr, 0,
                      stream);
    if (st != PKV_OK) return st;
  }
  st = hip_status(launch_paged_attn_partition(a), who);
  if (st != PKV_OK) return st;
  return hip_status(launch_paged_attn_merge(a), who);
}

// ---------------------------------------------------------------------------
// shared-prefix decode
// ---------------------------------------------------------------------------
extern "C" size_t pkv_paged_attn_shared_prefix_workspace_bytes(int kv_dtype, int num_seqs, int num_q_heads,
                                                               int num_kv_heads, int head_dim, int max_seq_len,
                                                               int prefix_blocks, int partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || prefix_blocks < 0) return 0;
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads) return 0;
  const int suffix = max_seq_len - prefix_blocks * 16;
  const size_t split = pkv_paged_attn_workspace_bytes(kv_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                      suffix > 0 ? suffix : 0, partition_size);
  // prefix records, whole-sequence records, then the decode's plan area and
  // split records (the plan area alone when no sequence can be cut)
  return prefix_area_bytes(num_seqs, num_q_heads, head_dim) +
         whole_record_area_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim) +
         (split > 0 ? split : plan_area_bytes(num_seqs));
}

extern "C" pkv_status pkv_paged_attn_decode_shared_prefix(
    void* out, const void* query, int q_dtype, void* k_cache, void* v_cache, int kv_dtype, const void* key,
    const void* value, const int32_t* positions, int32_t* slot_mapping_out, const int32_t* block_tables,
    int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int block_size, int num_blocks, float sm_scale, int prefix_blocks, int partition_size, unsigned flags,
    void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "pkv_paged_attn_decode_shared_prefix";
  if (kv_dtype != q_dtype || (kv_dtype != PKV_BF16 && kv_dtype != PKV_F16))
    return fail(PKV_EUNSUPPORTED, "%s: built for bf16 / f16 caches of the query dtype", who);
  if (prefix_blocks < 1 || prefix_blocks > max_blocks_per_seq)
    return fail(PKV_EINVAL, "%s: prefix_blocks must lie in [1, max_blocks_per_seq]", who);
  if (key && (!value || !positions)) return fail(PKV_EINVAL, "%s: key given without value or positions", who);
  if (num_seqs > 0 && (long long)num_seqs * max_blocks_per_seq >= (1LL << 29))
    return fail(PKV_EUNSUPPORTED, "%s: batch too large (num_seqs * max_blocks_per_seq >= 2^29)", who);
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_EINVAL, "%s: negative or zero size", who);
  pkv_status st = check_cache_shape(who, block_size, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if (num_q_heads % num_kv_heads) return fail(PKV_EINVAL, "%s: num_q_heads %% num_kv_heads != 0", who);
  if (num_q_heads / num_kv_heads > 16)
    return fail(PKV_EUNSUPPORTED, "%s: query group size above 16 is not built", who);
  if (flags & ~(unsigned)PKV_DECODE_STREAM_KV) return fail(PKV_EINVAL, "%s: unknown flags 0x%x", who, flags);
  const size_t pre_bytes = num_seqs > 0 ? prefix_area_bytes(num_seqs, num_q_heads, head_dim) +
                                              whole_record_area_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim)
                                        : 0;
  if (num_seqs > 0) {
    if (!workspace || workspace_bytes < pre_bytes)
      return fail(PKV_EWORKSPACE, "%s: workspace of at least %zu bytes needed, %zu given", who, pre_bytes,
                  workspace_bytes);
    if (((uintptr_t)workspace) & 127) return fail(PKV_EINVAL, "%s: workspace must be 128-byte aligned", who);
    if (!block_tables) return fail(PKV_EINVAL, "%s: null pointer argument", who);
  }
  // the suffix decode: tables from entry prefix_blocks on, lengths past the prefix
  AttnArgs a = fill_args(out, query, q_dtype, k_cache, v_cache, kv_dtype, nullptr, nullptr,
                         block_tables ? block_tables + prefix_blocks : nullptr, max_blocks_per_seq - prefix_blocks,
                         seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, sm_scale,
                         partition_size, 0, 0, flags, stream);
  a.table_stride = max_blocks_per_seq;
  a.len_off = prefix_blocks * block_size;
  a.prefix = (const float*)workspace;
  a.srec = workspace ? (float*)((char*)workspace + prefix_area_bytes(num_seqs, num_q_heads, head_dim)) : nullptr;
  if (key) {
    a.new_k = key;
    a.new_v = value;
    a.positions = positions;
    a.slots_out = slot_mapping_out;
  }
  st = prepare_attn(a, who, workspace ? (char*)workspace + pre_bytes : nullptr,
                               workspace_bytes > pre_bytes ? workspace_bytes - pre_bytes : 0, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  if (check_env()) {
    st = device_check(block_tables, max_blocks_per_seq, seq_lens, num_seqs, block_size, num_blocks, nullptr, 0,
                      stream);
    if (st != PKV_OK) return st;
    std::vector<int32_t> bt((size_t)num_seqs * max_blocks_per_seq), sl(num_seqs);
    hipStream_t hs = (hipStream_t)stream;
    int e = hipMemcpyAsync(bt.data(), block_tables, bt.size() * 4, hipMemcpyDeviceToHost, hs);
    e |= hipMemcpyAsync(sl.data(), seq_lens, sl.size() * 4, hipMemcpyDeviceToHost, hs);
    e |= hipStreamSynchronize(hs);
    if (e != hipSuccess) return fail(PKV_EHIP, "PKV_CHECK: copying tables to the host failed");
    st = pkv_validate_shared_prefix(bt.data(), max_blocks_per_seq, sl.data(), num_seqs, block_size, prefix_blocks);
    if (st != PKV_OK) return st;
  }
  // The shared blocks are sequence 0's first prefix_blocks entries.  The
  // prefix items run in the decode's own launch, on workgroups dispatched
  // after its slots, in the compute units its workgroups leave; without
  // four waves per workgroup (fewer than 4 KV heads) the prefix pass runs
  // first on its own.
  const int pfx_wgs = prefix_workgroups(num_seqs, num_q_heads, num_kv_heads, device_cu_count());
  if (pfx_wgs > 0) {
    st = hip_status(launch_shared_prefix_decode(a, block_tables, prefix_blocks, (float*)workspace, pfx_wgs), who);
  } else {
    st = hip_status(launch_prefix_attn(query, q_dtype, k_cache, v_cache, block_tables, prefix_blocks,
                                       (float*)workspace, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                                       sm_scale, stream),
                    who);
    if (st != PKV_OK) return st;
    st = hip_status(launch_paged_attn_partition(a), who);
  }
  if (st != PKV_OK) return st;
  return hip_status(launch_paged_attn_merge(a), who);
}

extern "C" size_t pkv_quest_scratch_bytes(int num_seqs, int num_kv_heads, int max_blocks_per_seq) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0) return 0;
  return align256((size_t)num_seqs * num_kv_heads * max_blocks_per_seq * 8);
}

extern "C" pkv_status pkv_quest_summarize(const void* k_cache, int kv_dtype, void* k_summary,
                                          const int32_t* block_tables, int max_blocks_per_seq,
                                          const int32_t* seq_lens, int num_seqs, int num_blocks, int block_size,
                                          int num_kv_heads, int head_dim, int last_only, void* stream) {
  const char* who = "pkv_quest_summarize";
  pkv_status st = check_cache_shape(who, block_size, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if (kv_dtype != PKV_BF16 && kv_dtype != PKV_F16) return fail(PKV_EUNSUPPORTED, "%s: cache must be bf16 or f16", who);
  if (num_seqs < 0 || max_blocks_per_seq < 0 || num_blocks < 0) return fail(PKV_EINVAL, "%s: negative size", who);
  if (num_seqs == 0 || max_blocks_per_seq == 0) return PKV_OK;
  if (!last_only && max_blocks_per_seq > 65535)
    return fail(PKV_EUNSUPPORTED, "%s: max_blocks_per_seq above 65535 needs last_only", who);
  if (!k_cache || !k_summary || !block_tables || !seq_lens) return fail(PKV_EINVAL, "%s: null pointer", who);
  return hip_status(launch_quest_summarize(k_cache, kv_dtype, k_summary, block_tables, max_blocks_per_seq, seq_lens,
                                           num_seqs, num_blocks, num_kv_heads, head_dim, last_only ? 1 : 0, stream),
                    who);
}

extern "C" pkv_status pkv_quest_select(const void* query, int q_dtype, const void* k_summary,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* seq_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int num_blocks, int budget_blocks,
                                       int32_t* selected, void* scratch, size_t scratch_bytes, void* stream) {
  const char* who = "pkv_quest_select";
  pkv_status st = check_cache_shape(who, block_size, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if (q_dtype != PKV_BF16 && q_dtype != PKV_F16) return fail(PKV_EUNSUPPORTED, "%s: query must be bf16 or f16", who);
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads) return fail(PKV_EINVAL, "%s: num_q_heads %% num_kv_heads", who);
  if (num_q_heads / num_kv_heads > 16) return fail(PKV_EUNSUPPORTED, "%s: query group size above 16", who);
  if (budget_blocks <= 0) return fail(PKV_EINVAL, "%s: budget_blocks must be positive", who);
  if (num_seqs < 0 || max_blocks_per_seq < 0 || num_blocks < 0) return fail(PKV_EINVAL, "%s: negative size", who);
  if (num_seqs == 0) return PKV_OK;
  if ((long long)num_seqs * num_kv_heads > 2147483647LL || max_blocks_per_seq / 16 >= 65535)
    return fail(PKV_EUNSUPPORTED, "%s: shape too large", who);
  const size_t need = pkv_quest_scratch_bytes(num_seqs, num_kv_heads, max_blocks_per_seq);
  if (!scratch || scratch_bytes < need)
    return fail(PKV_EWORKSPACE, "%s: scratch of %zu bytes needed, %zu given", who, need, scratch_bytes);
  if (((uintptr_t)scratch) & 7) return fail(PKV_EINVAL, "%s: scratch must be 8-byte aligned", who);
  if (!query || !k_summary || !block_tables || !seq_lens || !selected) return fail(PKV_EINVAL, "%s: null pointer", who);
  return hip_status(launch_quest_select(query, q_dtype, k_summary, block_tables, max_blocks_per_seq, seq_lens,
                                        num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, budget_blocks,
                                        selected, scratch, stream),
                    who);
}

extern "C" pkv_status pkv_paged_attn_merge(void* out, int q_dtype, const int32_t* seq_lens, int num_seqs,
                                           int num_q_heads, int num_kv_heads, int head_dim, int max_seq_len,
                                           int partition_size, int sink_tokens, int window_tokens,
                                           const void* workspace, size_t workspace_bytes, void* stream) {
  if (max_seq_len < 0 || max_seq_len % 16) return fail(PKV_EINVAL, "pkv_paged_attn_merge: bad max_seq_len");
  if (sink_tokens < 0 || window_tokens < 0) return fail(PKV_EINVAL, "pkv_paged_attn_merge: negative sink/window");
  return run_attn(false, true, out, nullptr, q_dtype, nullptr, nullptr, q_dtype, nullptr, nullptr, nullptr,
                  max_seq_len / 16, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, 16, 0, 1.f,
                  partition_size, sink_tokens, window_tokens, 0u, const_cast<void*>(workspace), workspace_bytes,
                  stream);
}

// ---------------------------------------------------------------------------
// cache writes
// ---------------------------------------------------------------------------
extern "C" pkv_status pkv_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* seq_ids, const int32_t* positions, int num_tokens,
                                       int num_seqs, int block_size, int num_blocks, void* stream) {
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 0 || block_size <= 0 || num_blocks < 0)
    return fail(PKV_EINVAL, "pkv_slot_mapping: bad size");
  if (num_tokens == 0) return PKV_OK;
  if (!slot_mapping || !block_tables || !positions) return fail(PKV_EINVAL, "pkv_slot_mapping: null pointer");
  if (!seq_ids && num_tokens > num_seqs)
    return fail(PKV_EINVAL, "pkv_slot_mapping: without seq_ids, token j belongs to sequence j < num_seqs");
  return hip_status(launch_slot_mapping(slot_mapping, block_tables, max_blocks_per_seq, seq_ids, positions,
                                        num_tokens, num_seqs, block_size, num_blocks, stream),
                    "pkv_slot_mapping");
}

extern "C" pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                            int dtype, const int32_t* slot_mapping, int num_tokens, int num_blocks,
                                            int block_size, int num_kv_heads, int head_dim, void* stream) {
  pkv_status st = check_cache_shape("pkv_reshape_and_cache", block_size, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if (!is_float_storage(dtype))
    return fail(PKV_EUNSUPPORTED, "pkv_reshape_and_cache: dtype must be f32, bf16 or f16");
  if (num_tokens < 0 || num_blocks < 0) return fail(PKV_EINVAL, "pkv_reshape_and_cache: negative size");
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_EINVAL, "pkv_reshape_and_cache: null pointer");
  if (check_env()) {
    st = device_check(nullptr, 0, nullptr, 0, block_size, num_blocks, slot_mapping, num_tokens, stream);
    if (st != PKV_OK) return st;
  }
  return hip_status(launch_reshape_and_cache(key, value, k_cache, v_cache, dtype_bytes(dtype), slot_mapping,
                                             num_tokens, num_blocks, block_size, num_kv_heads, head_dim, stream),
                    "pkv_reshape_and_cache");
}

extern "C" pkv_status pkv_append_kv(const void* key, const void* value, void* k_cache, void* v_cache, int dtype,
                                    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_ids,
                                    const int32_t* positions, int32_t* slot_mapping, int num_tokens, int num_seqs,
                                    int num_blocks, int block_size, int num_kv_heads, int head_dim, void* stream) {
  pkv_status st = check_cache_shape("pkv_append_kv", block_size, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if (!is_float_storage(dtype)) return fail(PKV_EUNSUPPORTED, "pkv_append_kv: dtype must be f32, bf16 or f16");
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 0 || num_blocks < 0)
    return fail(PKV_EINVAL, "pkv_append_kv: negative size");
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !block_tables || !positions)
    return fail(PKV_EINVAL, "pkv_append_kv: null pointer");
  if (!seq_ids && num_tokens > num_seqs)
    return fail(PKV_EINVAL, "pkv_append_kv: without seq_ids, token j belongs to sequence j < num_seqs");
  return hip_status(launch_append_kv(key, value, k_cache, v_cache, dtype_bytes(dtype), block_tables,
                                     max_blocks_per_seq, seq_ids, positions, slot_mapping, num_tokens, num_seqs,
                                     num_blocks, block_size, num_kv_heads, head_dim, stream),
                    "pkv_append_kv");
}

extern "C" pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                                      const int32_t* src_dst, int n, int dtype, int num_blocks, int block_size,
                                      int num_kv_heads, int head_dim, void* stream) {
  pkv_status st = check_cache_shape("pkv_copy_blocks", block_size, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if (!dtype_bytes(dtype)) return fail(PKV_EUNSUPPORTED, "pkv_copy_blocks: unknown dtype");
  if (n < 0 || num_blocks < 0) return fail(PKV_EINVAL, "pkv_copy_blocks: negative size");
  if (n == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_dst) return fail(PKV_EINVAL, "pkv_copy_blocks: null pointer");
  if ((k_scales == nullptr) != (v_scales == nullptr))
    return fail(PKV_EINVAL, "pkv_copy_blocks: give both scale arrays or neither");
  // INT4 rows: head_dim / 2 bytes
  return hip_status(launch_copy_blocks(k_cache, v_cache, k_scales, v_scales, src_dst, n, dtype_bytes(dtype),
                                       num_blocks, block_size, num_kv_heads,
                                       dtype == PKV_I4 ? head_dim / 2 : head_dim, stream),
                    "pkv_copy_blocks");
}

extern "C" pkv_status pkv_append_kv_quantized(const void* key, const void* value, int src_dtype, void* k_tail,
                                              void* v_tail, void* k_codes, void* v_codes, int code_dtype,
                                              float* k_scales, float* v_scales, const int32_t* block_tables,
                                              int max_blocks_per_seq, const int32_t* positions, int num_seqs,
                                              int num_blocks, int block_size, int num_kv_heads, int head_dim,
                                              void* stream) {
  const char* who = "pkv_append_kv_quantized";
  pkv_status st = check_cache_shape(who, block_size, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if (!is_float_storage(src_dtype)) return fail(PKV_EUNSUPPORTED, "%s: source must be f32/bf16/f16", who);
  if (!is_code_storage(code_dtype))
    return fail(PKV_EUNSUPPORTED, "%s: codes must be i8, i4, fp8e4m3 or fp8e5m2", who);
  if (num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq < 0) return fail(PKV_EINVAL, "%s: negative size", who);
  if (num_seqs == 0) return PKV_OK;
  if (num_kv_heads > 65535) return fail(PKV_EUNSUPPORTED, "%s: shape too large", who);
  if (!key || !value || !k_tail || !v_tail || !k_codes || !v_codes || !k_scales || !v_scales || !block_tables ||
      !positions)
    return fail(PKV_EINVAL, "%s: null pointer", who);
  return hip_status(launch_append_quantized(key, value, src_dtype, k_tail, v_tail, k_codes, v_codes, code_dtype,
                                            k_scales, v_scales, nullptr, nullptr, block_tables, max_blocks_per_seq,
                                            positions, num_seqs, num_blocks, num_kv_heads, head_dim, stream),
                    who);
}

extern "C" pkv_status pkv_append_kv_quantized_grouped(
    const void* key, const void* value, int src_dtype, void* k_tail, void* v_tail, void* k_codes, void* v_codes,
    int code_dtype, float* k_tile_scales, float* k_channel_scales, float* v_token_scales,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* positions, int num_seqs, int num_blocks,
    int block_size, int num_kv_heads, int head_dim, void* stream) {
  const char* who = "pkv_append_kv_quantized_grouped";
  pkv_status st = check_cache_shape(who, block_size, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if (!is_float_storage(src_dtype)) return fail(PKV_EUNSUPPORTED, "%s: source must be f32/bf16/f16", who);
  if (!is_code_storage(code_dtype))
    return fail(PKV_EUNSUPPORTED, "%s: codes must be i8, i4, fp8e4m3 or fp8e5m2", who);
  if (num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq < 0) return fail(PKV_EINVAL, "%s: negative size", who);
  if (num_seqs == 0) return PKV_OK;
  if (num_kv_heads > 65535) return fail(PKV_EUNSUPPORTED, "%s: shape too large", who);
  if (!key || !value || !k_tail || !v_tail || !k_codes || !v_codes || !k_tile_scales || !k_channel_scales ||
      !v_token_scales || !block_tables || !positions)
    return fail(PKV_EINVAL, "%s: null pointer", who);
  return hip_status(launch_append_quantized(key, value, src_dtype, k_tail, v_tail, k_codes, v_codes, code_dtype,
                                            k_tile_scales, nullptr, k_channel_scales, v_token_scales, block_tables,
                                            max_blocks_per_seq, positions, num_seqs, num_blocks, num_kv_heads,
                                            head_dim, stream),
                    who);
}

extern "C" pkv_status pkv_quantize_kv_grouped(const void* src_cache, int src_dtype, void* dst_codes,
                                              int code_dtype, float* dst_tile_scales, float* dst_group_scales,
                                              int group, const int32_t* block_ids, int n_blocks, int num_blocks,
                                              int block_size, int num_kv_heads, int head_dim, void* stream) {
  const char* who = "pkv_quantize_kv_grouped";
  pkv_status st = check_cache_shape(who, block_size, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if (!is_float_storage(src_dtype)) return fail(PKV_EUNSUPPORTED, "%s: source must be f32/bf16/f16", who);
  if (!is_code_storage(code_dtype))
    return fail(PKV_EUNSUPPORTED, "%s: codes must be i8, i4, fp8e4m3 or fp8e5m2", who);
  if (group != PKV_GROUP_CHANNEL && group != PKV_GROUP_TOKEN) return fail(PKV_EINVAL, "%s: unknown group %d", who, group);
  if (n_blocks < 0 || num_blocks < 0) return fail(PKV_EINVAL, "%s: negative size", who);
  if (!block_ids && n_blocks > num_blocks) return fail(PKV_EINVAL, "%s: n_blocks > num_blocks", who);
  if (n_blocks == 0) return PKV_OK;
  if (!src_cache || !dst_codes || !dst_group_scales) return fail(PKV_EINVAL, "%s: null pointer", who);
  return hip_status(launch_quantize_kv_grouped(src_cache, src_dtype, dst_codes, code_dtype, dst_tile_scales,
                                               dst_group_scales, group, block_ids, n_blocks, num_blocks, num_kv_heads,
                                               head_dim, stream),
                    who);
}

extern "C" pkv_status pkv_quantize_kv(const void* src_cache, int src_dtype, void* dst_codes, int code_dtype,
                                      float* dst_scales, const int32_t* block_ids, int n_blocks, int num_blocks,
                                      int block_size, int num_kv_heads, int head_dim, void* stream) {
  pkv_status st = check_cache_shape("pkv_quantize_kv", block_size, num_kv_heads, head_dim);
  if (st != PKV_OK) return st;
  if (!is_float_storage(src_dtype)) return fail(PKV_EUNSUPPORTED, "pkv_quantize_kv: source must be f32/bf16/f16");
  if (!is_code_storage(code_dtype))
    return fail(PKV_EUNSUPPORTED, "pkv_quantize_kv: codes must be i8, i4, fp8e4m3 or fp8e5m2");
  if (n_blocks < 0 || num_blocks < 0) return fail(PKV_EINVAL, "pkv_quantize_kv: negative size");
  if (!block_ids && n_blocks > num_blocks) return fail(PKV_EINVAL, "pkv_quantize_kv: n_blocks > num_blocks");
  if (n_blocks == 0) return PKV_OK;
  if (!src_cache || !dst_codes || !dst_scales) return fail(PKV_EINVAL, "pkv_quantize_kv: null pointer");
  return hip_status(launch_quantize_kv(src_cache, src_dtype, dst_codes, code_dtype, dst_scales, block_ids, n_blocks,
                                       num_blocks, block_size, num_kv_heads, head_dim, stream),
                    "pkv_quantize_kv");
}
