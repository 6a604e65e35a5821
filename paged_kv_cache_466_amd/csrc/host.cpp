// Host-only parts of the C ABI: the thread-local error message and the
// checks of block tables, lengths and slots that run on host copies of them.
// Plain C++ (no HIP), so that it can also be built under the address and
// undefined-behaviour sanitizers with the pool and the prefix cache.
#include <stdarg.h>
#include <stdio.h>

#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = 0; }

pkv_status fail(pkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

}  // namespace pkv

using namespace pkv;

extern "C" const char* pkv_last_error(void) { return g_err; }
extern "C" const char* pkv_version(void) { return "pkv 0.2.0 (gfx950)"; }

extern "C" pkv_status pkv_validate_tables(const int32_t* block_tables, int max_blocks_per_seq,
                                          const int32_t* seq_lens, int num_seqs, int block_size, int num_blocks,
                                          const int32_t* slot_mapping, int num_tokens) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || block_size <= 0 || num_blocks < 0)
    return fail(PKV_EINVAL, "pkv_validate_tables: negative size");
  if (num_seqs > 0 && (!block_tables || !seq_lens))
    return fail(PKV_EINVAL, "pkv_validate_tables: null table");
  for (int s = 0; s < num_seqs; ++s) {
    const int L = seq_lens[s];
    if (L < 0 || (long long)L > (long long)max_blocks_per_seq * block_size)
      return fail(PKV_EINVAL, "seq_lens[%d] = %d outside [0, %d]", s, L, max_blocks_per_seq * block_size);
    const int nb = (L + block_size - 1) / block_size;
    for (int i = 0; i < nb; ++i) {
      const int b = block_tables[(size_t)s * max_blocks_per_seq + i];
      if (b < 0 || b >= num_blocks)
        return fail(PKV_EINVAL, "block_tables[%d][%d] = %d outside [0, %d)", s, i, b, num_blocks);
    }
  }
  if (slot_mapping && num_tokens > 0) {
    const long long nslots = (long long)num_blocks * block_size;
    std::vector<char> seen((size_t)nslots, 0);
    for (int j = 0; j < num_tokens; ++j) {
      const int sl = slot_mapping[j];
      if (sl < 0) continue;
      if (sl >= nslots) return fail(PKV_EINVAL, "slot_mapping[%d] = %d outside [0, %lld)", j, sl, nslots);
      if (seen[sl]) return fail(PKV_EINVAL, "slot_mapping[%d] = %d repeats an earlier slot", j, sl);
      seen[sl] = 1;
    }
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_validate_shared_prefix(const int32_t* block_tables, int max_blocks_per_seq,
                                                 const int32_t* seq_lens, int num_seqs, int block_size,
                                                 int prefix_blocks) {
  const char* who = "pkv_validate_shared_prefix";
  if (num_seqs < 0 || block_size <= 0 || prefix_blocks < 0 || prefix_blocks > max_blocks_per_seq)
    return fail(PKV_EINVAL, "%s: bad sizes", who);
  if (num_seqs > 0 && (!block_tables || !seq_lens)) return fail(PKV_EINVAL, "%s: null table", who);
  for (int s = 0; s < num_seqs; ++s) {
    if ((long long)seq_lens[s] < (long long)prefix_blocks * block_size)
      return fail(PKV_EINVAL, "%s: seq_lens[%d] = %d is shorter than the %d-token prefix", who, s, seq_lens[s],
                  prefix_blocks * block_size);
    for (int i = 0; i < prefix_blocks; ++i)
      if (block_tables[(size_t)s * max_blocks_per_seq + i] != block_tables[i])
        return fail(PKV_EINVAL, "%s: block_tables[%d][%d] = %d differs from sequence 0's %d", who, s, i,
                    block_tables[(size_t)s * max_blocks_per_seq + i], block_tables[i]);
  }
  return PKV_OK;
}
