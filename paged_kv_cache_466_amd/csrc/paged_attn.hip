// Paged decode attention for gfx950.
//
// The decode walks each sequence's physical blocks through its block table,
// in logical order ("Chapter 18", "How PagedAttention Works"; Learning-AI
// topic t13_4, block table; "KV Cache Engineering", section 10), scores the
// grouped query heads against each block's keys (GQA, "KV Cache Engineering"
// section 1: the G = Hq/Hkv query heads of a group read the same KV head),
// keeps an online softmax and accumulates P.V.  The tokens of a sequence are
// cut only at multiples of partition_size; a piece of a sequence either
// writes the final output (the whole sequence in one piece) or fp32 partials
// (m, l, acc) that a merge kernel combines by log-sum-exp.
//
// Kernels:
//  * paged_attn_wave_kernel - bf16 / f16 caches and INT8, INT4, FP8-E4M3 and
//    FP8-E5M2 codes (converted to a 16-bit type in registers).  Each
//    workgroup takes an equal run of the batch's partitions, or of its
//    blocks when partitions span several (stream-K style, crossing sequence
//    boundaries), and runs one wave per KV head over the same list of
//    physical blocks.  Per 16-token block: S^T = K Q^T on
//    v_mfma_f32_16x16x32 (K rows go straight from HBM into the A operand;
//    the query group, padded to 16 heads, is the B operand), then out^T +=
//    V^T P^T on v_mfma_f32_16x16x16, where the score tile already has the
//    B-operand layout and V^T is read from an LDS copy of the block with the
//    transposing ds_read_b64_tr_b16.  Blocks are loaded with buffer loads
//    into a ring of DEPTH register tiles, so DEPTH-1 blocks are in flight
//    per wave while one computes.  Rows outside the kept range and tiles past the end
//    are given an out-of-range buffer offset: the hardware returns zeros for
//    them without touching memory, which both masks poisoned slots (no
//    0 * NaN in the MFMA) and keeps the ring branch-free.
//  * paged_attn_simple_kernel - fp32 caches (and any group size): scores in
//    LDS, plain fp32 FMAs.  Exact fp32 arithmetic, for the fp32 path.
//  * paged_attn_merge_kernel - log-sum-exp combine of the partials (and,
//    after a shared prefix, of the prefix's record).
//  * prefix_attn_kernel - blocks every sequence of the batch shares,
//    attended once for all query rows (a dense product on the matrix cores),
//    leaving one record per (sequence, query head) for the merge.
//
// Scores are kept in the log2 domain: s2 = (q.k) * sm_scale * log2(e), so
// exp(s - m) = exp2(s2 - m2).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kBS = 16;                     // tokens per block
constexpr float kLog2e = 1.4426950408889634f;

constexpr int kPrefixWaves = 4;                // waves of a prefix item
constexpr int kPrefixCG = 3;                  // 16-row column groups per wave
constexpr int kPrefixRows = 16 * kPrefixCG;   // rows of a workgroup (every wave takes all of them)
constexpr int kPrefixTable = 2048;            // shared-block entries staged in LDS at a time

template <int D>
__host__ __device__ constexpr int prefix_lds_bytes() {
  return kPrefixWaves * kBS * (2 * D + 16) + kPrefixTable * 4 + kPrefixWaves * kPrefixRows * (D + 4) * 4;
}

// Shared-prefix pass: see prefix_attn_kernel.
struct PrefixParams {
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const int32_t* table;   // the shared physical blocks, in logical order
  float* rec;             // [S][Hq][D + 4]
  int num_prefix_blocks, num_seqs, num_q_heads, num_kv_heads, num_blocks;
  float scale_log2;
  int items;              // (row tile, KV head) items: row tiles x num_kv_heads
};

struct AttnParams {
  void* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const float* k_scales;
  const float* v_scales;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws;            // partial records (see AttnArgs)
  int* plan;            // wave path: per sequence (slot of its first record, first and last workgroup, 0)
  int rec_floats;       // floats per record
  int num_seqs, mbs, num_q_heads, num_kv_heads, num_blocks;
  int partition_size, num_partitions;
  int sink, window;
  int min_units;        // fewest units a workgroup takes
  int list_cap;         // blocks a workgroup's list holds
  int table_bytes;      // bytes of block_tables (of `selected` for a selected decode)
  const int32_t* selected;   // selected decode: [S][Hkv][budget] (physical, logical block)
  int budget;                // selected decode: pages per (sequence, KV head)
  int qtok;                  // query tokens per sequence (the last qtok positions, causal)
  const float* k_chan;       // grouped scales: K per (block, KV head, channel); v_scales per token
  // fused slot write (new_k != null): the new token of sequence s, key/value
  // [S][Hkv][D], goes to position positions[s] (< 0: none) before it is read;
  // its slot goes to slots_out[s] when slots_out != null
  const void* new_k;
  const void* new_v;
  const int32_t* positions;
  int32_t* slots_out;
  // Shared-prefix decode: block_tables starts at the first suffix entry of
  // row 0, rows are tstride entries apart (tstride = mbs otherwise), and a
  // sequence's length counts from token len_off.  srec (non-null only
  // then): one record per (sequence, KV head), where a sequence finished in
  // one piece leaves its record instead of its output; the merge combines
  // every sequence's records with the prefix's.
  int tstride;
  int len_off;
  float* srec;
  float scale_log2;     // sm_scale * log2(e)
  // combined shared-prefix launch: the first pfx_wgs workgroups along x
  // take the prefix items of pfx, the decode's workgroup slots follow them
  int pfx_wgs;
  PrefixParams pfx;
};

__device__ __forceinline__ int clamp_len(int L, int mbs) {
  const int cap = mbs * kBS;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Is logical token t taken into attention for a sequence of length L?
// (Evaluated without branches: bitwise, not short-circuit, operators.)
__device__ __forceinline__ bool kept(int t, int L, int sink, int window) {
  const bool all = (sink | window) == 0;
  return (t < L) & (all | (t < sink) | (t >= L - window));
}

// Kept length of sequence s: its tokens past len_off, at most mbs blocks.
__device__ __forceinline__ int seq_len_at(const AttnParams& p, int s) {
  return clamp_len(p.seq_lens[s] - p.len_off, p.mbs);
}

__device__ __forceinline__ int table_entry(const AttnParams& p, int s, int lb) {
  int pb = p.block_tables[(size_t)s * p.tstride + lb];
  // a bad table must not make the kernel leave the cache arrays
  return (pb < 0 || pb >= p.num_blocks) ? 0 : pb;
}


// ===========================================================================
// Wave kernel
// ===========================================================================

// The 16-bit type the MFMAs use: the query's for 16-bit and FP8 caches; f16
// for INT8 codes, which convert to f16 in two cheap steps (below).
template <typename QT, typename KVT>
struct MmaType { typedef QT type; };
template <typename QT>
struct MmaType<QT, I8> { typedef F16 type; };
template <typename QT>
struct MmaType<QT, I4> { typedef F16 type; };

// Two INT8 codes (bytes 2h, 2h+1 of w) -> two f16 values, exactly.  With
// u = c + 128 (the code's bits with the top bit flipped), the f16 with bits
// 0x64 << 8 | u is 1024 + u; subtracting 1152 leaves c.
template <int H>
__device__ __forceinline__ uint32_t i8x2_f16(uint32_t u) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  // bytes: u[2H], 0x64, u[2H+1], 0x64
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, H ? 0x04030402u : 0x04010400u);
  const h2 x = __builtin_bit_cast(h2, b) - h2{(_Float16)1152.0f, (_Float16)1152.0f};
  return __builtin_bit_cast(uint32_t, x);
}

// Eight INT4 codes (the nibbles of w, element 2i in the low nibble of byte
// i, two's complement) -> eight f16 values, exactly, in the interleaved order
// (0, 4, 1, 5, 2, 6, 3, 7): the nibbles at bits s and s + 16 of w >> s
// (s = 0, 4, 8, 12) are elements s/4 and s/4 + 4.  With u = code + 8 (bit 3
// of the nibble flipped), masking a pair of nibbles to bits 0-3 of each half,
// flipping bit 3 and setting the 0x64 byte is one three-input bit operation
// that leaves the f16 1024 + u; minus 1032 is the code.  The nibbles at bits
// 4-7 need no shift: in place they give 1024 + 16 u, and (1024 + 16 u) / 16 -
// 72 is the code, one packed FMA, exact.  Nine operations per eight codes;
// the query's elements and the staged V rows use the same order.
__device__ __forceinline__ uint4 i4x8_f16_il(uint32_t w) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  auto low = [](uint32_t x) {
    const uint32_t b = (x & 0x000F000Fu) ^ 0x64086408u;
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, b) - h2{(_Float16)1032.0f, (_Float16)1032.0f});
  };
  auto high = [](uint32_t x) {
    const uint32_t b = (x & 0x00F000F0u) ^ 0x64806480u;
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2, b),
                                                                  h2{(_Float16)0.0625f, (_Float16)0.0625f},
                                                                  h2{(_Float16)-72.0f, (_Float16)-72.0f}));
  };
  const uint32_t w8 = w >> 8;
  return make_uint4(low(w), high(w), low(w8), high(w8));
}

// (q0..q7) -> (q0, q4, q1, q5, q2, q6, q3, q7): 16-bit elements of a uint4
__device__ __forceinline__ uint4 interleave8(uint4 q) {
  return make_uint4(__builtin_amdgcn_perm(q.z, q.x, 0x05040100u), __builtin_amdgcn_perm(q.z, q.x, 0x07060302u),
                    __builtin_amdgcn_perm(q.w, q.y, 0x05040100u), __builtin_amdgcn_perm(q.w, q.y, 0x07060302u));
}

// 8 codes -> 8 elements of the MFMA type, exactly (every INT8 value is an f16
// value; every finite FP8-E4M3 and FP8-E5M2 value is a bf16 and an f16 value).
template <typename MT, typename KVT>
__device__ __forceinline__ uint4 to16(uint32_t w0, uint32_t w1) {
  typedef Mfma<MT> M;
  if constexpr (std::is_same<KVT, I8>::value) {
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
    return make_uint4(i8x2_f16<0>(u0), i8x2_f16<1>(u0), i8x2_f16<0>(u1), i8x2_f16<1>(u1));
  } else if constexpr (std::is_same<KVT, BF8>::value) {
    return make_uint4(M::template bf8x2<false>(w0), M::template bf8x2<true>(w0), M::template bf8x2<false>(w1),
                      M::template bf8x2<true>(w1));
  } else {
    return make_uint4(M::template fp8x2<false>(w0), M::template fp8x2<true>(w0), M::template fp8x2<false>(w1),
                      M::template fp8x2<true>(w1));
  }
}

// GRP: grouped scales (K per channel, V per token), whose per-lane scale
// loads ride in the ring too.
template <typename KVT, int D, bool GRP = false>
struct WaveCfg {
  static constexpr bool kCodes = KVT::bits < 16;
  static constexpr int NC = D / 32;                    // q.K MFMAs per block (k = 32)
  static constexpr int NN = D / 16;                    // P.V MFMAs per block (n = 16)
  static constexpr int ROW_BYTES = D * KVT::bits / 8;  // one token row of one KV head
  // 16-byte K loads per lane per block: codes take a quarter row per lane group
  static constexpr int KCH = kCodes ? ROW_BYTES / 4 / 16 : NC;
  static_assert(KCH >= 1, "a lane group's quarter row must fill a 16-byte load");
  static constexpr int LANES_PER_ROW = ROW_BYTES / 16;
  static constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;
  static constexpr int VCH = kBS / ROWS_PER_PASS;      // 16-byte V loads per lane per block
  // Ring of register tiles: one block in flight per wave while one computes,
  // eight waves per compute unit.  Deeper rings (3, 4, 6, 8) measured slower
  // for every cache type on the Llama-3-8B and 32K shapes and no faster at
  // 128K: a launch's first burst of loads, DEPTH blocks from every wave at
  // once, queues in front of the blocks the waves need first.
  static constexpr int DEPTH = 2;
  static constexpr int VROW = D * 2 + 16;              // LDS bytes per staged V row (16-bit, padded)
  // one staged V block, then (grouped) the D / 2 f16 pairs of channel factors
  static constexpr int VSTAGE = kBS * VROW + (GRP ? 2 * D : 0);
};

// d-offset (elements) of the 8-element k-chunk that lane group `kg` feeds to
// MFMA number `c` of the q.K product.  Any assignment works as long as K and
// Q use the same one; it is chosen so that each load instruction reads long
// contiguous runs: 16-bit rows read 64 contiguous bytes per row per
// instruction, 8-bit rows let one lane read 32 contiguous bytes.
template <typename KVT, int D>
__device__ __forceinline__ int qk_doff(int c, int kg) {
  if constexpr (KVT::bytes == 2) return 32 * c + 8 * kg;
  else return (D / 4) * kg + 8 * c;
}

// ===========================================================================
// Work split
//
// A "unit" is a partition (partition_size tokens from t = 0) that holds at
// least one kept token.  Numbering the units of all sequences one after the
// other gives U units.  With K workgroups along x, Q = max(min_units,
// ceil(U / K)) units per workgroup and K_eff = ceil(U / Q) workgroups at
// work, workgroup w takes units [w U / K_eff, (w + 1) U / K_eff): all get Q
// or Q - 1 units, and a range may begin or end inside a sequence and may
// cover several sequences.  A workgroup runs one wave per KV head of its
// group of heads; the waves walk the same list of physical blocks at the
// same time, each reading its head's rows.
//
// The part of a sequence inside one workgroup is a "segment".  A whole
// sequence is finished where it is; otherwise each wave writes a partial
// record: slot 2w for the workgroup's first segment, 2w + 1 for its last (a
// segment between the two always holds its whole sequence).  The workgroup
// holding a sequence's first unit leaves in the plan area, for the merge,
// the slot of that first record and the first and last workgroups the
// sequence reaches; every later workgroup's record of it sits in its slot 2w.
// ===========================================================================
struct SeqUnits {
  int np;   // partitions covering the sequence
  int a;    // units [0, a) hold sink tokens
  int b0;   // units [a, n) are partitions b0 .. np-1 (window tokens)
  int n;    // units
};

__device__ __forceinline__ SeqUnits seq_units(int L, int psize, int sink, int window) {
  SeqUnits u;
  u.np = (L + psize - 1) / psize;
  if ((sink | window) == 0) {
    u.a = u.b0 = u.n = u.np;
    return u;
  }
  u.a = min(u.np, (min(sink, L) + psize - 1) / psize);
  u.b0 = window > 0 ? min(u.np, max(u.a, max(0, L - window) / psize)) : u.np;
  u.n = u.a + (u.np - u.b0);
  return u;
}
__device__ __forceinline__ int unit_partition(const SeqUnits& u, int i) { return i < u.a ? i : u.b0 + (i - u.a); }

__device__ __forceinline__ int lane_scan_incl(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// 64 consecutive sequences, lane i describing sequence s0 + i.
// Positions in the split are measured in units, or in blocks (`weighted`):
// then a workgroup's share is a run of blocks, and it takes the units that
// start inside it (see build_block_list).
struct SeqWindow {
  int s0;      // first sequence (uniform)
  int base;    // position of its first unit (uniform)
  int total;   // units (blocks when weighted) in the window (uniform)
  int L;       // this lane's clamped length
  int n;       // its units
  int P;       // position of its first unit
};

// SEL: a selected decode, whose units are the selected pages (at most
// `budget` blocks of the sequence).
template <bool SEL>
__device__ __forceinline__ SeqWindow load_window(const AttnParams& p, int s0, int base, int lane,
                                                 bool weighted) {
  SeqWindow w;
  w.s0 = s0;
  w.base = base;
  const int s = s0 + lane;
  w.L = s < p.num_seqs ? seq_len_at(p, s) : 0;
  if constexpr (SEL) w.n = min(p.budget, (w.L + kBS - 1) / kBS);
  else w.n = seq_units(w.L, p.partition_size, p.sink, p.window).n;
  const int wt = weighted ? (w.L + kBS - 1) / kBS : w.n;
  const int incl = lane_scan_incl(wt, lane);
  w.P = base + incl - wt;
  w.total = __builtin_amdgcn_readlane(incl, 63);
  return w;
}

// Blocks of units [i0, i1) of a sequence of length L, in logical order:
// blocks lb_begin .. lb_begin + n_a - 1, then b0 .. b0 + (n_need - n_a) - 1
// (the blocks between hold no kept token).
struct SegBlocks {
  int lb_begin, n_a, b0, n_need;
};

__device__ __forceinline__ SegBlocks segment_blocks(const AttnParams& p, int L, int i0, int i1) {
  const SeqUnits su = seq_units(L, p.partition_size, p.sink, p.window);
  const int t_begin = unit_partition(su, i0) * p.partition_size;
  const int t_end = min((unit_partition(su, i1 - 1) + 1) * p.partition_size, L);
  SegBlocks b;
  b.lb_begin = t_begin / kBS;
  const int lb_end = (t_end + kBS - 1) / kBS;
  int a1 = lb_end, b0 = lb_end;
  if ((p.sink | p.window) != 0) {
    const int sink_end = min(lb_end, (p.sink + kBS - 1) / kBS);   // blocks holding a sink token
    a1 = max(b.lb_begin, sink_end);
    b0 = p.window > 0 ? min(lb_end, max(max(b.lb_begin, max(0, L - p.window) / kBS), a1)) : lb_end;
  }
  b.n_a = a1 - b.lb_begin;
  b.b0 = b0;
  b.n_need = b.n_a + (lb_end - b0);
  return b;
}

constexpr int kMaxWavesPerGroup = 8;   // KV heads per workgroup
constexpr int kQueryLds = 6144;        // LDS bytes per wave for the queries of its first segments
constexpr int kMaxQuerySegs = 64;      // segments whose sequence number is kept for that
constexpr int kEndKey = -1;            // key of the list entry after the last block

// LDS of a workgroup of `waves` waves: per wave a V staging area and a query
// area, then the block list (list_cap entries and the end entry), the
// sequences of the first segments, four counters, and the sequences whose
// last unit the workgroup holds (at most one per list entry).
__host__ __device__ constexpr int wave_group_lds(int vstage, int waves, int list_cap) {
  return waves * (vstage + kQueryLds) + (list_cap + 1) * 16 + kMaxQuerySegs * 4 + 16 + list_cap * 4;
}

// Writes the workgroup's block list into LDS (one wave calls it).  Entry k:
// (the block's physical number, gathered from the table in one round of
// loads once the list is written - for a selected decode the byte offset of
// its selection entry, which differs per KV head -, first token of the block
// with bit 31 set when some
// token of the block is masked for some query, length of its sequence,
// segment key); the key packs the sequence (bits 8+), the
// segment's number in the workgroup (bits 2-7, saturating), whether its
// record goes to slot 2w + 1 (bit 1) and whether it is the whole sequence
// (bit 0).  Also zeroes an empty sequence's output and writes the plan
// entries of the sequences that start here.
template <bool SEL, bool PFX>
__device__ __forceinline__ void build_block_list(const AttnParams& p, int head_dim, int lane, int4* list, int* segs,
                                                 int* counts, int* ends) {
  const int S = p.num_seqs;
  const int w = blockIdx.x;
  // workgroup s of the first head group zeroes sequence s when it is empty
  // (16-bit outputs: zero bits are zero); with a shared prefix its output is
  // the prefix's, written by the kernel
  if (blockIdx.y == 0 && w < S && seq_len_at(p, w) == 0) {
    if (!p.srec) {
      const int n16 = p.num_q_heads * p.qtok * head_dim / 8;
      uint4* o = reinterpret_cast<uint4*>(p.out) + (size_t)w * n16;
      for (int i = lane; i < n16; i += 64) o[i] = make_uint4(0, 0, 0, 0);
    }
    // nothing for the merge to do
    if (p.plan && lane == 0) reinterpret_cast<int4*>(p.plan)[w] = make_int4(0, 0, 0, 0);
  }

  // Weighted split: a full-attention decode whose partitions span several
  // blocks balances blocks rather than partitions.  The units of a 128K
  // sequence and one appended token are 256 partitions of 32 blocks and one
  // of 1 block; counted as units, 4 such sequences over 256 workgroups give
  // some workgroups 5 partitions (160 blocks), counted in blocks none gets
  // more than 129.  A unit starting inside a workgroup's run of blocks
  // belongs to it whole, so a workgroup reads at most step - 1 blocks past
  // its run: the host sizes the grid for that, and step is kept small
  // enough next to the block list (3 step <= list_cap).
  const int bpp = p.partition_size / kBS;
  const bool weighted = !SEL && (p.sink | p.window) == 0 && bpp > 1 && 3 * bpp <= p.list_cap;
  const int step = weighted ? bpp : 1;   // position step between a sequence's units
  SeqWindow win = load_window<SEL>(p, 0, 0, lane, weighted);
  int U = win.total;
  for (int s0 = 64; s0 < S; s0 += 64) U += load_window<SEL>(p, s0, U, lane, weighted).total;
  int nb = 0, nseg = 0, nend = 0;
  if (U > 0) {
    // a combined launch's prefix workgroups follow the decode's slots
    const int K = PFX ? (int)gridDim.x - p.pfx_wgs : (int)gridDim.x;
    int k_eff;
    if (weighted) {
      // every run at least one unit long (so that every workgroup between a
      // sequence's first and last holds a unit of it) and min_units long
      k_eff = max(1, min(K, min(U / (p.min_units * step), U / step)));
    } else {
      const int Q = max(p.min_units, (U + K - 1) / K);
      k_eff = (U + Q - 1) / Q;
    }
    // floor(a * b / c) for a * b <= K * U: in 32 bits when that fits (every
    // shape but the largest; a 64-bit division is several times longer)
    const bool narrow = (unsigned long long)K * (unsigned)U < (1ull << 32);
    auto muldiv = [&](int a, int b, int c) {
      return narrow ? (int)((unsigned)a * (unsigned)b / (unsigned)c) : (int)((long long)a * b / c);
    };
    if (w < k_eff) {
      const int u0 = muldiv(w, U, k_eff);
      const int u1 = muldiv(w + 1, U, k_eff);
      if (S > 64) {
        win = load_window<SEL>(p, 0, 0, lane, weighted);
        while (win.base + win.total <= u0 && win.s0 + 64 < S)
          win = load_window<SEL>(p, win.s0 + 64, win.base + win.total, lane, weighted);
      }
      // the first sequence with a unit starting at or past u0 (weighted, it
      // may lie in the next window)
      const unsigned long long hit = __ballot(win.n > 0 && win.P + (win.n - 1) * step >= u0);
      int s = hit ? win.s0 + (int)__ffsll((long long)hit) - 1 : min(win.s0 + 64, S);
      while (s < S) {
        if (s >= win.s0 + 64) win = load_window<SEL>(p, win.s0 + 64, win.base + win.total, lane, weighted);
        const int l = s - win.s0;
        const int n = __builtin_amdgcn_readlane(win.n, l);
        const int P = __builtin_amdgcn_readlane(win.P, l);
        const int L = __builtin_amdgcn_readlane(win.L, l);
        if (P >= u1) break;
        // the units starting in [u0, u1): unit i starts at P + i step
        // (one-block units, step 1, skip the divisions)
        const int i0 = min(n, u0 > P ? (step == 1 ? u0 - P : (u0 - P + step - 1) / step) : 0);
        const int i1 = min(n, step == 1 ? u1 - P : (u1 - P + step - 1) / step);
        if (i0 < i1) {
          SegBlocks sb;
          if constexpr (SEL) {
            // units are entries i0 .. i1-1 of the sequence's selection
            sb.lb_begin = i0;
            sb.n_a = sb.n_need = i1 - i0;
            sb.b0 = 0;
          } else {
            sb = segment_blocks(p, L, i0, i1);
          }
          const int whole = (i0 == 0 && i1 == n) ? 1 : 0;
          const int upper = nseg > 0 ? 1 : 0;   // not the workgroup's first segment
          const int key = (s << 8) | (min(nseg, 63) << 2) | (upper << 1) | whole;
          // the grid is sized so that every range fits; the bound only
          // keeps a wrong size from writing past the list
          const int cnt = min(sb.n_need, p.list_cap - nb);
          const bool windowed = (p.sink | p.window) != 0;
          for (int j = lane; j < cnt; j += 64) {
            const int lb = j < sb.n_a ? sb.lb_begin + j : sb.b0 + (j - sb.n_a);
            // masked: past L - T (the first query token's last position), or
            // partly outside the keep-mask
            const int t0 = lb * kBS;
            const bool masked = (t0 + kBS - 1 > L - p.qtok) |
                                (windowed & (t0 + kBS > p.sink) & (t0 < L - p.window));
            // SEL: offset of the selection entry (KV head 0); the block's
            // first token comes with the entry
            list[nb + j] = SEL ? make_int4((s * p.num_kv_heads * p.budget + lb) * 8, 0, L, key)
                               : make_int4((s * p.tstride + lb) * 4, t0 | (masked ? (int)0x80000000u : 0), L, key);
          }
          if (lane == 0 && nseg < kMaxQuerySegs) segs[nseg] = s;
          // the workgroup holding a sequence's last unit writes its new token
          if (p.new_k && i1 == n && cnt > 0) {
            if (lane == 0) ends[nend] = s;
            ++nend;
          }
          if (i0 == 0 && p.plan && blockIdx.y == 0 && lane == 0) {
            // the workgroup whose run holds the start of the last unit
            const int w_last = narrow ? (int)(((unsigned)(P + (n - 1) * step + 1) * (unsigned)k_eff - 1u) / (unsigned)U)
                                      : (int)(((long long)(P + (n - 1) * step + 1) * k_eff - 1) / U);
            // w: 1 when a whole sequence left its record in srec
            reinterpret_cast<int4*>(p.plan)[s] = make_int4(2 * w + upper, w, w_last, p.srec && w_last == w ? 1 : 0);
          }
          nb += cnt;
          ++nseg;
        }
        ++s;
      }
    }
  }
  if constexpr (!SEL) {
    // the table entries of the whole list in one round of loads: entry .x
    // becomes the physical block (the same for every KV head)
    const __amdgpu_buffer_rsrc_t tabr = make_rsrc(p.block_tables, p.table_bytes);
    for (int j0 = lane; j0 < nb; j0 += 4 * 64) {
      int pbv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + 64 * q;
        pbv[q] = (int)__builtin_amdgcn_raw_buffer_load_b32(tabr, j < nb ? list[j].x : kOutOfRange, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (j0 + 64 * q < nb) list[j0 + 64 * q].x = pbv[q];
    }
  }
  if (lane == 0) {
    list[nb] = make_int4(kOutOfRange, 0, 0, kEndKey);
    counts[0] = nb;
    counts[1] = nseg;
    counts[2] = nend;
  }
}

template <typename QT, int D, int DEPTH>
__device__ __forceinline__ void prefix_item(const PrefixParams& p, int item);

// PFX: the combined shared-prefix launch.  The last pfx_wgs workgroups
// along x take the prefix items (prefix_item, on their first four waves,
// items strided over all of them).  They are dispatched after every decode
// slot, so they take the compute units the decode's workgroups leave.
template <typename QT, typename KVT, int D, bool STREAM, bool SEL, bool GRP, bool PFX = false>
__global__ __launch_bounds__(64 * kMaxWavesPerGroup) __attribute__((amdgpu_waves_per_eu(2)))
void paged_attn_wave_kernel(AttnParams p) {
  if constexpr (PFX) {
    const int first = (int)gridDim.x - p.pfx_wgs;
    if ((int)blockIdx.x >= first) {
      if (threadIdx.x >= 64 * kPrefixWaves) return;   // the barriers count the waves still running
      const int stride = p.pfx_wgs * (int)gridDim.y;
      for (int item = (int)blockIdx.x - first + p.pfx_wgs * (int)blockIdx.y; item < p.pfx.items; item += stride)
        prefix_item<QT, D, 2>(p.pfx, item);   // a shorter ring: the decode's register budget
      return;
    }
  }
  typedef WaveCfg<KVT, D, GRP> C;
  static_assert(!GRP || (C::kCodes && std::is_same<typename MmaType<QT, KVT>::type, F16>::value && !SEL),
                "grouped scales are built for integer codes, without a selection");
  typedef typename MmaType<QT, KVT>::type MT;
  typedef Mfma<MT> M;     // operands of both products
  typedef Mfma<QT> MO;    // the output type
  constexpr int NC = C::NC, NN = C::NN, KCH = C::KCH, VCH = C::VCH, DEPTH = C::DEPTH;
  constexpr bool kCodes = C::kCodes;
  // INT4: key and value elements come out of the conversion interleaved
  // within each group of 8 (i4x8_f16_il): the query operand is interleaved to
  // match, and the staged V rows hold interleaved columns, put back in order
  // when the results leave LDS
  constexpr bool kIL = KVT::bits == 4;
  // the query is rescaled into f16 (INT8 caches with a bf16 query)
  constexpr bool kRescaleQ = !std::is_same<MT, QT>::value;
  // Scores may exceed the running max by this much (log2 units) before the
  // accumulators are rescaled: probabilities stay below 2^8.
  constexpr float kSlack = 8.0f;
  constexpr int kQRegs = kQueryLds / 1024;   // 16-byte query loads per lane

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int waves = blockDim.x >> 6;
  const int kvh = blockIdx.y * waves + wave;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int T = p.qtok;
  // Columns of S^T / out^T: (query token t, head gh of the group), col =
  // t * G + gh, NCOL = G * T <= 16.  col / G as (col * inv_g) >> 16, exact
  // for col < 16 and every G <= 16.
  const int NCOL = G * T;
  const int inv_g = 0x10000 / G + 1;
  const int g = lane & 15;       // this lane's column
  const int kg = lane >> 4;      // lane group: k-chunk of the operands, 4-row slab of outputs
  const int lane_t = g < NCOL ? (g * inv_g) >> 16 : 0;   // its query token
  // query / output row of column col of sequence s
  auto qrow = [&](size_t s, int col) {
    const int t = (col * inv_g) >> 16;
    return (s * T + t) * p.num_q_heads + kvh * G + (col - t * G);
  };
  uint8_t* vstage = lds + wave * C::VSTAGE;
  uint8_t* qlds = lds + waves * C::VSTAGE + wave * kQueryLds;
  int4* list = reinterpret_cast<int4*>(lds + waves * (C::VSTAGE + kQueryLds));
  int* segs = reinterpret_cast<int*>(list + p.list_cap + 1);
  int* counts = segs + kMaxQuerySegs;
  int* ends = counts + 4;

  if (wave == 0) build_block_list<SEL, PFX>(p, D, lane, list, segs, counts, ends);
  __syncthreads();
  if (kvh >= p.num_kv_heads) return;
  const int nb = __builtin_amdgcn_readfirstlane(counts[0]);
  const int nseg = __builtin_amdgcn_readfirstlane(counts[1]);

  if (!SEL && !kCodes && p.new_k) {
    // Fused slot write: the new token of every sequence whose last unit this
    // workgroup holds (the only workgroup reading that block).  Each wave
    // writes its own head's key and value rows, and its stores complete
    // before it loads any block.
    const int nend = __builtin_amdgcn_readfirstlane(counts[2]);
    constexpr int CH = D / 8;   // 16-byte pieces of a 16-bit row
    for (int j = 0; j < nend; ++j) {
      const int s = __builtin_amdgcn_readfirstlane(ends[j]);
      const int pos_abs = p.positions[s];
      if (pos_abs < 0) continue;
      const int pos = pos_abs - p.len_off;   // len_off is whole blocks
      if (pos < 0 || pos / kBS >= p.mbs) continue;
      const int pb = p.block_tables[(size_t)s * p.tstride + pos / kBS];
      if (pb < 0 || pb >= p.num_blocks) continue;
      const size_t slot = (size_t)pb * kBS + pos % kBS;
      if (lane < 2 * CH) {
        const bool isv = lane >= CH;
        const int c = isv ? lane - CH : lane;
        const uint4 v =
            reinterpret_cast<const uint4*>(isv ? p.new_v : p.new_k)[((size_t)s * p.num_kv_heads + kvh) * CH + c];
        uint4* cache = reinterpret_cast<uint4*>(const_cast<void*>(isv ? p.v_cache : p.k_cache));
        cache[(slot * p.num_kv_heads + kvh) * CH + c] = v;
      }
      if (p.slots_out && blockIdx.y == 0 && wave == 0 && lane == 0) p.slots_out[s] = (int)slot;
    }
    // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left alone): the rows are in
    // memory before this wave issues its first block load
    if (nend > 0) __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  // queries of the first segments, copied to LDS at the start of the ring
  const int q_chunks = NCOL * D / 8;                   // 16-byte pieces of one segment's query columns
  const int q_segs = min(min(kQueryLds / (NCOL * D * 2), kMaxQuerySegs), nseg);

  // block-list entry k (the end entry for k >= nb), wave-uniform
  auto entry_at = [&](int k) {
    const int4 r = list[min(k, nb)];
    return make_int4(__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                     __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(r.w));
  };
  // (physical block, logical block) of a list entry: the physical block the
  // list already holds, or this head's selection entry for a selected decode
  // (per head, so loaded here)
  const __amdgpu_buffer_rsrc_t tab = make_rsrc(SEL ? (const void*)p.selected : (const void*)p.block_tables,
                                               p.table_bytes);
  const int sel_head = kvh * p.budget * 8;
  auto load_table = [&](int off) {
    if constexpr (SEL) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(tab, off + sel_head, 0, 0));
      return make_int2((int)v[0], (int)v[1]);
    } else {
      return make_int2(off, 0);   // the list entry holds the physical block
    }
  };
  // first token of an entry's block, and whether some token of it is
  // masked for some query (a selected decode has one query token and no
  // keep-mask)
  auto block_start = [&](const int2& ent, const int4& e) {
    return SEL ? (int)__builtin_amdgcn_readfirstlane(ent.y) * kBS : (e.y & 0x7fffffff);
  };
  auto block_masked = [&](int t0, const int4& e) { return SEL ? t0 + kBS > e.z : e.y < 0; };

  struct Tile {
    uint4 k[KCH];
    uint4 v[VCH];
    float ks, vs;
    float kc[2];           // grouped: the two channel scales of this lane's factor pair
    floatx4 vts;           // grouped: token scales of rows 4 kg .. 4 kg + 3
    int t0;   // first token of the block
  };
  const int row_stride = p.num_kv_heads * C::ROW_BYTES;        // bytes between token rows
  const int krow = lane & 15;
  const int kcol = kCodes ? (C::ROW_BYTES / 4) * kg : 16 * kg;   // bytes
  const int k_off = krow * row_stride + kcol;
  // This head's rows of block 0.  Block b starts b * kBS * Hkv * ROW_BYTES
  // bytes further on, which is (b * Hkv * 4) << kTileShift: the byte offset
  // of its scale row, shifted.
  const uint8_t* k_head = reinterpret_cast<const uint8_t*>(p.k_cache) + (size_t)kvh * C::ROW_BYTES;
  const uint8_t* v_head = reinterpret_cast<const uint8_t*>(p.v_cache) + (size_t)kvh * C::ROW_BYTES;
  constexpr int kTileShift = __builtin_ctz(kBS * C::ROW_BYTES / 4);
  static_assert((kBS * C::ROW_BYTES / 4) == (1 << kTileShift), "tile bytes must be a power of two");
  const uint32_t scale_row_bytes = (uint32_t)p.num_kv_heads * 4;
  // the scales of this head in every block (num_blocks * Hkv * 4 < 2^31,
  // checked on the host); an empty pool reads nothing
  const int sbytes = kCodes && p.num_blocks > 0 ? p.num_blocks * (int)scale_row_bytes - kvh * 4 : 0;
  const __amdgpu_buffer_rsrc_t ks_r = make_rsrc(p.k_scales + kvh, sbytes);
  // grouped: token scales [block][head][16] (num_blocks * Hkv * 64 < 2^31,
  // checked on the host), channel scales [block][head][D]
  const __amdgpu_buffer_rsrc_t vs_r =
      GRP ? make_rsrc(p.v_scales + kvh * kBS, p.num_blocks > 0 ? (p.num_blocks * p.num_kv_heads - kvh) * kBS * 4 : 0)
          : make_rsrc(p.v_scales + kvh, sbytes);
  const uint8_t* kchan_head = reinterpret_cast<const uint8_t*>(p.k_chan + (size_t)kvh * D);
  // grouped: lane l < D / 2 turns two channel scales (bytes kc_off and
  // kc_off + kc_step of the tile's row) into f16 factor pair l.  A lane
  // group's pairs (D / 8 of them, from pair D / 8 * kg) are the factors of
  // its quarter row in the order the key operand uses: channels (2m, 2m + 1)
  // of the quarter, or, with INT4's interleaved elements, (8c + i, 8c + i + 4)
  // for pair m = 4c + i.
  int kc_off = kOutOfRange, kc_step = 4;
  if constexpr (GRP) {
    if (lane < D / 2) {
      const int quarter = lane / (D / 8), m = lane % (D / 8);
      const int ch = kIL ? quarter * (D / 4) + 8 * (m / 4) + (m % 4) : 2 * lane;
      kc_off = 4 * ch;
      kc_step = kIL ? 16 : 4;
    }
  }
  int v_off[VCH], v_row[VCH];
#pragma unroll
  for (int ps = 0; ps < VCH; ++ps) {
    v_row[ps] = ps * C::ROWS_PER_PASS + lane / C::LANES_PER_ROW;
    v_off[ps] = v_row[ps] * row_stride + (lane % C::LANES_PER_ROW) * 16;
  }
  const int tile_bytes = p.num_blocks > 0 ? (kBS - 1) * row_stride + C::ROW_BYTES : 0;
  // Rows shorter than a 128-byte line (INT4 at head_dim 128, 8-bit codes at
  // 64) put two KV heads in each line, read by two waves of the workgroup:
  // they keep the default policy (a non-temporal line may be gone before
  // the second read)
  constexpr int kPol = (STREAM && C::ROW_BYTES % 128 == 0) ? kPolicyStream : 0;

  // e: list entry of the block, ent: its (physical, logical) block
  auto load_tile = [&](Tile& t, const int2& ent, const int4& e) {
    const bool valid = e.w != kEndKey;
    uint32_t pb = __builtin_amdgcn_readfirstlane(ent.x);
    pb = pb < (uint32_t)p.num_blocks ? pb : 0u;   // a bad table must not leave the cache arrays
    const uint32_t so = pb * scale_row_bytes;    // < 2^31: checked on the host
    const uint64_t tile = (uint64_t)so << kTileShift;
    const int nbytes = valid ? tile_bytes : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k_head + tile, nbytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v_head + tile, nbytes);
    const int t0 = block_start(ent, e);
    const int L = e.z;
    t.t0 = t0;
    // K rows that are not kept load as they are: their scores are masked
#pragma unroll
    for (int c = 0; c < KCH; ++c)
      t.k[c] = buf_load16<kPol>(kr, k_off + (kCodes ? 16 : 64) * c);
    // V rows that are not kept read as zeros (a zero weight times a NaN row
    // would still poison the product)
    int vo[VCH];
#pragma unroll
    for (int ps = 0; ps < VCH; ++ps) vo[ps] = v_off[ps];
    if (block_masked(t0, e)) {
#pragma unroll
      for (int ps = 0; ps < VCH; ++ps)
        if (!kept(t0 + v_row[ps], L, p.sink, p.window)) vo[ps] = kOutOfRange;
    }
#pragma unroll
    for (int ps = 0; ps < VCH; ++ps) t.v[ps] = buf_load16<kPol>(vr, vo[ps]);
    if constexpr (GRP) {
      t.ks = buf_load4(ks_r, 0, (int)so);
      const __amdgpu_buffer_rsrc_t cr = make_rsrc(kchan_head + (uint64_t)so * D, valid ? D * 4 : 0);
      t.kc[0] = buf_load4(cr, kc_off);
      t.kc[1] = buf_load4(cr, kc_off + kc_step);
      t.vts = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(vs_r, 16 * kg, (int)so * kBS, 0));
    } else if constexpr (kCodes) {
      t.ks = buf_load4(ks_r, 0, (int)so);
      t.vs = buf_load4(vs_r, 0, (int)so);
    } else {
      t.ks = t.vs = 1.f;
    }
  };

  // ---- per-segment state ---------------------------------------------------
  int cur_key = kEndKey;         // segment being accumulated
  typename M::vec8 qop[NC];      // query group as the B operand of S^T = K Q^T (zero rows for g >= G)
  float qfactor = p.scale_log2;  // log2-domain score factor of this lane's head (times the block's K scale)
  float m2 = -INFINITY;          // running max (log2 domain) of head g, same in all lane groups
  float lsum = 0.f;              // this lane's share of the softmax denominator
  floatx4 acc[NN];

  auto start_segment = [&](int key) {
    const int ord = (key >> 2) & 63;
    uint4 v[NC];
    if (ord < q_segs) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        v[c] = g < NCOL ? *reinterpret_cast<const uint4*>(qlds + (size_t)ord * NCOL * D * 2 +
                                                          (g * D + qk_doff<KVT, D>(c, kg)) * 2)
                        : make_uint4(0, 0, 0, 0);
    } else {
      const size_t row = qrow((size_t)(key >> 8), g < NCOL ? g : 0);
#pragma unroll
      for (int c = 0; c < NC; ++c)
        v[c] = g < NCOL ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.query) + row * D +
                                                          qk_doff<KVT, D>(c, kg))
                        : make_uint4(0, 0, 0, 0);
    }
    if constexpr (!kRescaleQ) {
#pragma unroll
      for (int c = 0; c < NC; ++c) qop[c] = __builtin_bit_cast(typename M::vec8, v[c]);
    } else {
      // bf16 -> f16 with the head's values scaled by 2^e so that the largest
      // lands in [2^14, 2^15): every bf16 value within 2^29 of the largest
      // stays exact, and the scores get 2^-e back through the factor
      float qf[NC][8];
      float mx = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        decode16<BF16>(v[c], qf[c]);
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(qf[c][i]));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      int e = 0;
      if (mx > 0.f) e = min(100, max(-100, 15 - __builtin_amdgcn_frexp_expf(mx)));
      qfactor = ldexpf(p.scale_log2, -e);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint4 w;
        w.x = M::pack2(ldexpf(qf[c][0], e), ldexpf(qf[c][1], e));
        w.y = M::pack2(ldexpf(qf[c][2], e), ldexpf(qf[c][3], e));
        w.z = M::pack2(ldexpf(qf[c][4], e), ldexpf(qf[c][5], e));
        w.w = M::pack2(ldexpf(qf[c][6], e), ldexpf(qf[c][7], e));
        qop[c] = __builtin_bit_cast(typename M::vec8, w);
      }
    }
    if constexpr (kIL) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        qop[c] = __builtin_bit_cast(typename M::vec8, interleave8(__builtin_bit_cast(uint4, qop[c])));
    }
    m2 = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int n = 0; n < NN; ++n) acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
  };

  // Results of the segment with this key.  Lane (g, kg) holds
  // out[g][16n + 4kg + i], i = 0..3.  The accumulators go through LDS (the
  // wave's V staging area, idle between blocks), 8 heads at a time, so that
  // every global store writes whole, contiguous 128-byte lines.
  auto finish_segment = [&](int key) {
    const bool whole = (key & 1) != 0;
    const size_t seq = (size_t)(key >> 8);
    float l = lsum + __shfl_xor(lsum, 16, 64);
    l += __shfl_xor(l, 32, 64);
    constexpr int RSTRIDE = D + 4;                      // floats per padded LDS row
    static_assert((8 * RSTRIDE + 32) * 4 <= C::VSTAGE, "result staging must fit the V staging area");
    float* rl = reinterpret_cast<float*>(vstage);
    // a whole sequence writes its output, or after a shared prefix its
    // record for the merge; a piece writes a record
    const bool to_out = whole && !p.srec;
    const float scale_out = to_out ? (l > 0.f ? 1.f / l : 0.f) : 1.f;
    // acc[NCOL][D], then m[16], l[16]
    float* rec = whole ? (p.srec ? p.srec + (seq * p.num_kv_heads + kvh) * p.rec_floats : nullptr)
                       : (p.ws ? p.ws + ((size_t)(2 * blockIdx.x + ((key >> 1) & 1)) * p.num_kv_heads + kvh) *
                                            p.rec_floats
                               : nullptr);
    for (int h0 = 0; h0 < NCOL; h0 += 8) {
      const int nh = min(8, NCOL - h0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (g >= h0 && g < h0 + 8) {
#pragma unroll
        for (int n = 0; n < NN; ++n)
          *reinterpret_cast<floatx4*>(rl + (g - h0) * RSTRIDE + 16 * n + 4 * kg) = acc[n] * scale_out;
      }
      if (h0 == 0 && kg == 0) {
        rl[8 * RSTRIDE + g] = m2;
        rl[8 * RSTRIDE + 16 + g] = l;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (to_out) {
        // nh output rows of D elements (rows of one query token are
        // contiguous): 8 elements per lane-store
        constexpr int CPR = D / 8;
        for (int c = lane; c < nh * CPR; c += 64) {
          const float* src = rl + (c / CPR) * RSTRIDE + (c % CPR) * 8;
          const floatx4 lo = *reinterpret_cast<const floatx4*>(src);
          const floatx4 hi = *reinterpret_cast<const floatx4*>(src + 4);
          // interleaved columns: positions (0..7) hold elements (0, 4, 1, 5, 2, 6, 3, 7)
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + qrow(seq, h0 + c / CPR) * D + (c % CPR) * 8) =
              kIL ? make_uint4(MO::pack2(lo[0], lo[2]), MO::pack2(hi[0], hi[2]), MO::pack2(lo[1], lo[3]),
                               MO::pack2(hi[1], hi[3]))
                  : make_uint4(MO::pack2(lo[0], lo[1]), MO::pack2(lo[2], lo[3]), MO::pack2(hi[0], hi[1]),
                               MO::pack2(hi[2], hi[3]));
        }
      } else if (whole || p.ws) {
        if constexpr (kIL) {
          constexpr int CPR = D / 8;
          for (int c = lane; c < nh * CPR; c += 64) {
            const float* src = rl + (c / CPR) * RSTRIDE + (c % CPR) * 8;
            const floatx4 lo = *reinterpret_cast<const floatx4*>(src);
            const floatx4 hi = *reinterpret_cast<const floatx4*>(src + 4);
            float* dst = rec + (size_t)h0 * D + 8 * c;
            *reinterpret_cast<floatx4*>(dst) = floatx4{lo[0], lo[2], hi[0], hi[2]};
            *reinterpret_cast<floatx4*>(dst + 4) = floatx4{lo[1], lo[3], hi[1], hi[3]};
          }
        } else {
          constexpr int CPR = D / 4;
          for (int c = lane; c < nh * CPR; c += 64)
            *reinterpret_cast<floatx4*>(rec + (size_t)h0 * D + 4 * c) =
                *reinterpret_cast<const floatx4*>(rl + (c / CPR) * RSTRIDE + (c % CPR) * 4);
        }
        if (h0 == 0 && lane < 8)
          *reinterpret_cast<floatx4*>(rec + (size_t)NCOL * D + 4 * lane) =
              *reinterpret_cast<const floatx4*>(rl + 8 * RSTRIDE + 4 * lane);
      }
    }
  };

  auto process = [&](const Tile& t, const int4& e, uint8_t* vst) {
    if (e.w != cur_key) {
      // a new segment: the previous one's results leave first (they are
      // staged through the V area this block is about to use)
      if (cur_key != kEndKey) finish_segment(cur_key);
      start_segment(e.w);
      cur_key = e.w;
    }
    const int t0 = t.t0, L = e.z;

    if constexpr (GRP) {
      const float r = t.ks > 0.f ? __builtin_amdgcn_rcpf(t.ks) : 0.f;
      if (lane < D / 2)
        *reinterpret_cast<uint32_t*>(vst + kBS * C::VROW + 4 * lane) = M::pack2(t.kc[0] * r, t.kc[1] * r);
    }
    // ---- V rows -> LDS (masked rows arrive as zeros) -----------------------
#pragma unroll
    for (int ps = 0; ps < VCH; ++ps) {
      const int cchunk = lane % C::LANES_PER_ROW;
      if constexpr (!kCodes) {
        *reinterpret_cast<uint4*>(vst + v_row[ps] * C::VROW + cchunk * 16) = t.v[ps];
      } else if constexpr (KVT::bits == 4) {
        // 32 codes -> 64 bytes of f16
        uint8_t* dst = vst + v_row[ps] * C::VROW + cchunk * 64;
        *reinterpret_cast<uint4*>(dst) = i4x8_f16_il(t.v[ps].x);
        *reinterpret_cast<uint4*>(dst + 16) = i4x8_f16_il(t.v[ps].y);
        *reinterpret_cast<uint4*>(dst + 32) = i4x8_f16_il(t.v[ps].z);
        *reinterpret_cast<uint4*>(dst + 48) = i4x8_f16_il(t.v[ps].w);
      } else {
        *reinterpret_cast<uint4*>(vst + v_row[ps] * C::VROW + cchunk * 32) = to16<MT, KVT>(t.v[ps].x, t.v[ps].y);
        *reinterpret_cast<uint4*>(vst + v_row[ps] * C::VROW + cchunk * 32 + 16) =
            to16<MT, KVT>(t.v[ps].z, t.v[ps].w);
      }
    }

    // ---- S^T = K Q^T --------------------------------------------------------
    floatx4 sacc = floatx4{0.f, 0.f, 0.f, 0.f};
    // grouped: channel factors s_d / s_tile in (0, 1] as f16 pairs (the tile
    // scale goes into the score factor), written to LDS before the V rows and
    // read back after them: 8 channels of k-chunk c per 4 pairs
    uint32_t kf[GRP ? 4 * NC : 1];
    if constexpr (GRP) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int m = 0; m < 4 * NC; m += 4) {
        const uint4 f = *reinterpret_cast<const uint4*>(vst + kBS * C::VROW + 4 * ((D / 8) * kg + m));
        kf[m] = f.x, kf[m + 1] = f.y, kf[m + 2] = f.z, kf[m + 3] = f.w;
      }
    }
    auto kscale = [&](uint4 k8, int c) {
      if constexpr (GRP) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const uint32_t w[4] = {k8.x, k8.y, k8.z, k8.w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, w[i]) * __builtin_bit_cast(h2, kf[4 * c + i]));
        return make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        return k8;
      }
    };
    if constexpr (!kCodes) {
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc = M::qk(__builtin_bit_cast(typename M::vec8, t.k[c]), qop[c], sacc);
    } else if constexpr (KVT::bits == 4) {
      // each 16-byte load holds 32 codes: four k-chunks of 8
#pragma unroll
      for (int c2 = 0; c2 < KCH; ++c2) {
        const uint32_t w[4] = {t.k[c2].x, t.k[c2].y, t.k[c2].z, t.k[c2].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc = M::qk(__builtin_bit_cast(typename M::vec8, kscale(i4x8_f16_il(w[j]), 4 * c2 + j)), qop[4 * c2 + j],
                       sacc);
      }
    } else {
#pragma unroll
      for (int c2 = 0; c2 < KCH; ++c2) {
        sacc = M::qk(__builtin_bit_cast(typename M::vec8, kscale(to16<MT, KVT>(t.k[c2].x, t.k[c2].y), 2 * c2)),
                     qop[2 * c2], sacc);
        sacc = M::qk(__builtin_bit_cast(typename M::vec8, kscale(to16<MT, KVT>(t.k[c2].z, t.k[c2].w), 2 * c2 + 1)),
                     qop[2 * c2 + 1], sacc);
      }
    }
    const float factor = qfactor * t.ks;
    // lane holds tokens 4*kg + i of this block for column g
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = sacc[i] * factor;
    // query token t sees positions up to L - T + t: blocks reaching past
    // L - T are masked per column
    const bool msk = block_masked(t0, e);
    if (msk) {
      const int lim = L - T + lane_t;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = t0 + 4 * kg + i;
        if (!kept(pos, L, p.sink, p.window) | (pos > lim)) sc[i] = -INFINITY;
      }
    }
    const float lm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    // ---- online softmax, rescaling only when a score passes m2 + slack -----
    // A column may have seen no visible position yet (m2 = -inf) and see
    // none in this block either: with several query tokens, a segment can
    // start at a block past a column's causal limit.  Such a column keeps
    // alpha = 1 and weights 0 (exp2(-inf - -inf) would be NaN), as an empty
    // partition does in the log-sum-exp merge.
    if (__ballot(lm > m2 + kSlack)) {
      float bmax = fmaxf(lm, __shfl_xor(lm, 16, 64));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
      const float mnew = fmaxf(m2, bmax);
      const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m2 - mnew);   // 0 while m2 = -inf
      lsum *= alpha;
#pragma unroll
      for (int n = 0; n < NN; ++n) acc[n] *= alpha;
      m2 = mnew;
    }
    // only a masked block can hold a column whose scores are all -inf
    const float mb = (msk & (m2 == -INFINITY)) ? 0.f : m2;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(sc[i] - mb);
    // P^T as the B operand (tokens 4kg..4kg+3 of head g), V scale folded in
    float vsc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vsc[i] = GRP ? t.vts[i] : t.vs;
    const uint32_t p01 = M::pack2(pr[0] * vsc[0], pr[1] * vsc[1]);
    const uint32_t p23 = M::pack2(pr[2] * vsc[2], pr[3] * vsc[3]);
    // the denominator sums the weights the MFMA uses (16-bit rounded), so
    // they add up to one; with codes the V scale is not part of the weight
    if constexpr (!kCodes) lsum = M::acc2(p23, M::acc2(p01, lsum));
    else lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const shortx4 pop = __builtin_bit_cast(shortx4, make_uint2(p01, p23));

    // ---- out^T += V^T P^T: V^T chunks through the transposing LDS read ----
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane i of each 16-lane group reads row 4kg + i/4, columns 4(i%4)..+3
    const uint8_t* rd = vst + (4 * kg + (g >> 2)) * C::VROW + (g & 3) * 8;
#pragma unroll
    for (int n = 0; n < NN; ++n) acc[n] = M::pv(M::tr_read(rd + n * 32), pop, acc[n]);
  };

  // ---- main loop: a ring of DEPTH tiles; block k + DEPTH is requested as
  // soon as block k's registers are free.  A selected decode fetches each
  // selection entry DEPTH steps before its tile load, so that the entry is
  // older than every load still in flight and no wait stalls the ring.
  // Loads past the end of the list read nothing.
  {
    Tile ring[DEPTH];
    int2 tab_ent[DEPTH];
    // entries k and k + DEPTH of slot d's next iteration: each list entry is
    // read from LDS once, 2 DEPTH blocks ahead (where a selected decode loads
    // its selection entry), and carried to its tile load and its processing
    int4 c0[DEPTH], c1[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) c0[d] = entry_at(d), c1[d] = entry_at(DEPTH + d);
    {
      int2 first[DEPTH];
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) first[d] = load_table(c0[d].x);
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) tab_ent[d] = load_table(c1[d].x);
      // The queries' loads overlap a selected decode's first selection
      // entries (no wait comes between them).  Branch-free, so that the
      // waits stay counted: pieces past the end load sequence 0's query and
      // land in unused LDS.
      // c / q_chunks as (c * inv) >> 16: exact for c < 6 * 64 and every
      // q_chunks = NCOL * D / 8 built (checked exhaustively on the host)
      const int inv = 0x10000 / q_chunks + 1;
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      u32x4 qv[kQRegs];
#pragma unroll
      for (int r = 0; r < kQRegs; ++r) {
        const int c = r * 64 + lane;
        const int i = (c * inv) >> 16;               // < kMaxQuerySegs: q_chunks >= 8
        const bool used = c < q_segs * q_chunks;
        const int si = segs[i];                      // read unconditionally, used only when set
        const int s = used ? si : 0;
        const int piece = used ? c - i * q_chunks : 0;
        // piece of column piece / (D / 8)
        qv[r] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.query) +
                                                qrow((size_t)s, piece / (D / 8)) * D + (piece % (D / 8)) * 8);
      }
#pragma unroll
      for (int r = 0; r < kQRegs; ++r) *reinterpret_cast<u32x4*>(qlds + (r * 64 + lane) * 16) = qv[r];
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) load_tile(ring[d], first[d], c0[d]);
    }
    __builtin_amdgcn_sched_barrier(0);
    for (int k0 = 0; k0 < nb; k0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int k = k0 + d;
        const int4 e0 = c0[d], e1 = c1[d], e2 = entry_at(k + 2 * DEPTH);
        c0[d] = e1;
        c1[d] = e2;
        if (k < nb) process(ring[d], e0, vstage);
        __builtin_amdgcn_sched_barrier(0);
        load_tile(ring[d], tab_ent[d], e1);
        tab_ent[d] = load_table(e2.x);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (cur_key != kEndKey) finish_segment(cur_key);
}

// ===========================================================================
// Simple fp32 kernel: scores in LDS, fp32 FMAs, chunks of 256 tokens with an
// online softmax across chunks.  Any group size with G * D <= 2048.
// ===========================================================================
template <typename QT, typename KVT, int D>
__global__ __launch_bounds__(256) void paged_attn_simple_kernel(AttnParams p) {
  constexpr int CH = 256;
  constexpr int MAXG = 16;
  constexpr int MAXPAIRS = MAXG * D / 256;
  __shared__ float qs[MAXG * D];
  __shared__ float sc[MAXG * CH];
  __shared__ float mrow[MAXG], lrow[MAXG], arow[MAXG];
  const int kvh = blockIdx.x, part = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int L = seq_len_at(p, s);
  const bool single = p.num_partitions == 1;
  const int t_begin = part * p.partition_size;
  const size_t head0 = (size_t)s * p.num_q_heads + kvh * G;
  if (t_begin >= L) {
    if (single && part == 0)
      for (int i = tid; i < G * D; i += 256) store_out<QT>(p.out, head0 * D + i, 0.f);
    return;
  }
  const int t_end = min(t_begin + p.partition_size, L);
  for (int i = tid; i < G * D; i += 256) qs[i] = load_elem<QT>(p.query, head0 * D + i);
  if (tid < G) {
    mrow[tid] = -INFINITY;
    lrow[tid] = 0.f;
  }
  float acc[MAXPAIRS];
#pragma unroll
  for (int k = 0; k < MAXPAIRS; ++k) acc[k] = 0.f;
  __syncthreads();

  const size_t row_elems = (size_t)p.num_kv_heads * D;
  for (int c0 = t_begin; c0 < t_end; c0 += CH) {
    // scores of this chunk
    {
      const int t = c0 + tid;
      if (t < t_end && kept(t, L, p.sink, p.window)) {
        const int pb = table_entry(p, s, t / kBS);
        const size_t row = ((size_t)pb * kBS + t % kBS) * row_elems + (size_t)kvh * D;
        float f = 1.f;
        if (KVT::bytes == 1) f = p.k_scales[(size_t)pb * p.num_kv_heads + kvh];
        for (int gg = 0; gg < G; ++gg) {
          float dot = 0.f;
          for (int d = 0; d < D; ++d) dot = fmaf(qs[gg * D + d], load_elem<KVT>(p.k_cache, row + d), dot);
          sc[gg * CH + tid] = dot * f * p.scale_log2;
        }
      } else {
        for (int gg = 0; gg < G; ++gg) sc[gg * CH + tid] = -INFINITY;
      }
    }
    __syncthreads();
    // chunk max, new running max, probabilities, chunk sum (one wave per head)
    {
      const int wv = tid >> 6, ln = tid & 63;
      for (int gg = wv; gg < G; gg += 4) {
        float mx = -INFINITY;
        for (int i = ln; i < CH; i += 64) mx = fmaxf(mx, sc[gg * CH + i]);
        mx = wave_max(mx);
        const float mold = mrow[gg];
        const float mnew = fmaxf(mold, mx);
        float sum = 0.f;
        for (int i = ln; i < CH; i += 64) {
          const float e = mnew == -INFINITY ? 0.f : exp2f(sc[gg * CH + i] - mnew);
          sc[gg * CH + i] = e;
          sum += e;
        }
        sum = wave_sum(sum);
        if (ln == 0) {
          const float a = mnew == -INFINITY ? 1.f : exp2f(mold - mnew);
          arow[gg] = a;
          lrow[gg] = lrow[gg] * a + sum;
          mrow[gg] = mnew;
        }
      }
    }
    __syncthreads();
    // P.V for the (head, dim) pairs this thread owns
#pragma unroll
    for (int k = 0; k < MAXPAIRS; ++k) {
      const int i = tid + 256 * k;
      if (i >= G * D) break;
      const int gg = i / D, d = i % D;
      float a = acc[k] * arow[gg];
      const int n = min(CH, t_end - c0);
      for (int j = 0; j < n; ++j) {
        const float pj = sc[gg * CH + j];
        if (pj == 0.f) continue;
        const int t = c0 + j;
        const int pb = table_entry(p, s, t / kBS);
        const size_t row = ((size_t)pb * kBS + t % kBS) * row_elems + (size_t)kvh * D;
        float v = load_elem<KVT>(p.v_cache, row + d);
        if (KVT::bytes == 1) v *= p.v_scales[(size_t)pb * p.num_kv_heads + kvh];
        a = fmaf(pj, v, a);
      }
      acc[k] = a;
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < MAXPAIRS; ++k) {
    const int i = tid + 256 * k;
    if (i >= G * D) break;
    const int gg = i / D, d = i % D;
    const float den = lrow[gg];
    if (single) {
      store_out<QT>(p.out, (head0 + gg) * D + d, den > 0.f ? acc[k] / den : 0.f);
    } else {
      float* rec = p.ws + (((size_t)s * p.num_kv_heads + kvh) * p.num_partitions + part) * p.rec_floats;
      rec[gg * D + d] = acc[k];
      if (d == 0) {
        rec[G * D + gg] = mrow[gg];
        rec[G * D + 16 + gg] = den;
      }
    }
  }
}

// ===========================================================================
// Merge of the wave kernel's records.  For each sequence cut over several
// workgroups and each record column (query head of a group, times query
// token), out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i over its
// records, one per workgroup it reaches.  Whole sequences were finished by
// their waves and empty ones zeroed: their plan entries name one workgroup,
// and their workgroups return at once.  After a shared prefix every
// sequence is merged here: the prefix's record of the head (acc[D], m, l at
// `prefix`) is one more term, a whole sequence's record is in `srec`
// (plan entry w = 1), and an empty one has the prefix's term alone.
// One workgroup per (sequence, KV head, group of cpw columns): the columns of
// one record sit next to each other, so a workgroup reads whole record rows.
// Its 256 threads take (column, 16-byte piece of the row) outputs; when
// those are fewer than 256, the records are shared out among `parts` thread
// groups whose partial sums meet in LDS.  Each thread folds its records in
// one pass with a running max, so that all its record loads are issued
// together right after the plan entry's.  cpw is chosen on the host so that
// the grid has about a thousand workgroups: most of a workgroup's time is
// the latency of a few dependent loads, hidden by having many in flight.
// ===========================================================================
template <typename QT, int D>
__global__ __launch_bounds__(256) void paged_attn_merge_kernel(void* out, const float* ws, const int* plan,
                                                               int rec_floats, int num_q_heads, int num_kv_heads,
                                                               int qtok, int cpw, const float* prefix,
                                                               const float* srec) {
  constexpr int V4 = D / 4;   // 16-byte pieces of an output row
  __shared__ float red[256];
  __shared__ floatx4 pnum[256];
  __shared__ float pden[256];
  const int s = blockIdx.x, kvh = blockIdx.y, col0 = blockIdx.z * cpw;
  const int tid = threadIdx.x;
  const int G = num_q_heads / num_kv_heads;
  const int NCOL = G * qtok;
  const int ncols = min(cpw, NCOL - col0);
  // thread (output o, part): records part, part + parts, ..., combined in one
  // pass with a running max (one round of loads after the plan entry); the
  // parts then meet in LDS
  const int outs = cpw * V4;          // <= 256 (cpw <= 256 / V4, checked on the host)
  const int parts = 256 / outs;
  const int o = tid % outs, part = tid / outs;
  const int c = o / V4, d4 = o % V4;
  const bool act = part < parts && c < ncols;
  const int col = col0 + c;
  // the prefix record of column c (a shared prefix goes with one query
  // token), loaded with the plan entry rather than after the records
  float pm = -INFINITY, pl = 0.f;
  floatx4 pa = floatx4{0.f, 0.f, 0.f, 0.f};
  if (prefix && part == 0 && act) {
    const float* pre = prefix + ((size_t)s * num_q_heads + kvh * G + col) * (D + 4);
    pm = pre[D];
    pl = pre[D + 1];
    pa = *reinterpret_cast<const floatx4*>(pre + 4 * d4);
  }
  // (slot of the first record, first workgroup, last workgroup)
  const int4 e = reinterpret_cast<const int4*>(plan)[s];
  const bool cut = e.z > e.y;
  if (!cut && !prefix) return;
  // records: cut, e.z - e.y + 1 of them; after a shared prefix, whole (one,
  // in srec) or empty (none)
  const int np = cut ? e.z - e.y + 1 : e.w;
  // record i: slot e.x for i = 0, then slot 2 (e.y + i) of each later workgroup
  auto rec_of = [&](int i) {
    if (!cut) return srec + ((size_t)s * num_kv_heads + kvh) * rec_floats;
    const int slot = i == 0 ? e.x : 2 * (e.y + i);
    return ws + ((size_t)slot * num_kv_heads + kvh) * rec_floats;
  };

  floatx4 num = floatx4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f, mrun = -INFINITY;
  // folds a term (m, l, acc) into (mrun, den, num); a term with m = -inf
  // (an empty piece) weighs nothing
  auto fold = [&](float mi, float li, const floatx4& a) {
    const float mn = fmaxf(mrun, mi);
    const float keep = mrun == -INFINITY ? 0.f : exp2f(mrun - mn);
    const float w = mi == -INFINITY ? 0.f : exp2f(mi - mn);
    num = num * keep + w * a;
    den = den * keep + w * li;
    mrun = mn;
  };
  if (act) {
    constexpr int U = 4;   // records in flight per thread
    int i = part;
    for (; i + (U - 1) * parts < np; i += U * parts) {
      float mi[U], li[U];
      floatx4 a[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float* r = rec_of(i + u * parts);
        mi[u] = r[NCOL * D + col];
        li[u] = r[NCOL * D + 16 + col];
        a[u] = *reinterpret_cast<const floatx4*>(r + col * D + 4 * d4);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) fold(mi[u], li[u], a[u]);
    }
    for (; i < np; i += parts) {
      const float* r = rec_of(i);
      fold(r[NCOL * D + col], r[NCOL * D + 16 + col], *reinterpret_cast<const floatx4*>(r + col * D + 4 * d4));
    }
  }
  if (parts > 1) {
    pnum[tid] = num;
    pden[tid] = den;
    red[tid] = mrun;
    __syncthreads();
    if (part == 0) {
      for (int j = 1; j < parts; ++j) fold(red[j * outs + o], pden[j * outs + o], pnum[j * outs + o]);
    }
  }
  if (part == 0 && act) {
    if (prefix) fold(pm, pl, pa);
    const int t = col / G, h = kvh * G + col % G;
    const size_t oi = (((size_t)s * qtok + t) * num_q_heads + h) * D + 4 * d4;
#pragma unroll
    for (int k = 0; k < 4; ++k) store_out<QT>(out, oi + k, den > 0.f ? num[k] / den : 0.f);
  }
}

// ===========================================================================
// Merge of the fp32 kernel's per-partition records: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p over the
// partitions p < ceil(L / partition_size); every such partition wrote its
// record (m = -inf, l = 0, acc = 0 when it kept no token).  One workgroup
// per (query head, sequence): the max first, then 8 partition rows at a time,
// each read by D/4 threads with 16-byte loads, 4 rows per thread in flight.
// ===========================================================================
template <typename QT, int D>
__global__ __launch_bounds__(256) void paged_attn_merge_units_kernel(void* out, const int32_t* seq_lens, const float* ws,
                                                               int rec_floats, int num_q_heads, int num_kv_heads,
                                                               int num_partitions, int partition_size, int max_len) {
  constexpr int TPR = D / 4;               // threads per partition row
  constexpr int ROWS = 256 / TPR;
  constexpr int U = 4;
  __shared__ float red[256];
  __shared__ floatx4 part_num[ROWS][TPR];
  __shared__ float part_den[ROWS];
  const int h = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x;
  const int G = num_q_heads / num_kv_heads;
  const int kvh = h / G, g = h % G;
  int L = seq_lens[s];
  L = L < 0 ? 0 : (L > max_len ? max_len : L);
  const int np = (L + partition_size - 1) / partition_size;
  // record of partition i: rec0 + i * rec_floats; acc row g, then m[16], l[16]
  const float* rec0 = ws + ((size_t)s * num_kv_heads + kvh) * num_partitions * rec_floats;
  const float* m_of = rec0 + (size_t)G * D + g;
  const float* l_of = m_of + 16;
  const float* a_of = rec0 + (size_t)g * D;
  float mx = -INFINITY;
  for (int i = tid; i < np; i += 256) mx = fmaxf(mx, m_of[(size_t)i * rec_floats]);
  red[tid] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float M = red[0];
  const int row = tid / TPR, c = tid % TPR;
  floatx4 num = floatx4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
    int i = row;
    for (; i + (U - 1) * ROWS < np; i += U * ROWS) {
      float mi[U], li[U];
      floatx4 a[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t r = (size_t)(i + u * ROWS) * rec_floats;
        mi[u] = m_of[r];
        li[u] = l_of[r];
        a[u] = *reinterpret_cast<const floatx4*>(a_of + r + 4 * c);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float e = exp2f(mi[u] - M);   // 0 for an empty partition
        num += e * a[u];
        den += e * li[u];
      }
    }
    for (; i < np; i += ROWS) {
      const size_t r = (size_t)i * rec_floats;
      const float e = exp2f(m_of[r] - M);
      num += e * *reinterpret_cast<const floatx4*>(a_of + r + 4 * c);
      den += e * l_of[r];
    }
  }
  part_num[row][c] = num;
  if (c == 0) part_den[row] = den;
  __syncthreads();
  if (tid < TPR) {
    floatx4 n = floatx4{0.f, 0.f, 0.f, 0.f};
    float dn = 0.f;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      n += part_num[r][tid];
      dn += part_den[r];
    }
    const size_t o = ((size_t)s * num_q_heads + h) * D + 4 * tid;
#pragma unroll
    for (int k = 0; k < 4; ++k) store_out<QT>(out, o + k, dn > 0.f ? n[k] / dn : 0.f);
  }
}

// ===========================================================================
// Shared-prefix pass
//
// When every sequence of a batch starts with the same P physical blocks (a
// prompt stored once and shared through the block tables: prefix caching,
// "KV Cache Engineering" section 11; copy-on-write forks, Learning-AI topic
// t13_4), the scores of the batch's S*G query rows of one KV head against
// those blocks are one dense product, Q [S*G, D] x K^T [D, 16 P], followed
// by P.V over the same blocks.  This pass reads each shared block once per
// 48 rows instead of once per sequence.  A workgroup of four waves takes 48
// rows of one KV head (row r is sequence r / G, head r % G of the group) and
// each wave a quarter of the blocks (48 rows do the pass in about a quarter
// fewer CU-microseconds than 32: an item's time is mostly per block).  Workgroup n takes KV head n % Hkv:
// consecutive workgroups go to the eight XCDs in turn, so with Hkv dividing
// or a multiple of 8 every XCD serves whole heads and one head's shared
// blocks stay in one XCD's L2 for all of its row tiles.  Per block a wave
// computes S^T = K Q^T for each of its three 16-row column groups from one K
// tile in registers (v_mfma_f32_16x16x32), and out^T += V^T P^T for all
// three from one transposed read of the V tile (v_mfma_f32_16x16x16).  The four waves' online-softmax
// states are combined in LDS by log-sum-exp into one record per (sequence,
// query head): acc[D] (unnormalised), m (log2 domain), l.  The suffix decode
// folds these records into its own results.
// ===========================================================================


// One item: 48 rows of one KV head against every shared block, on the
// first four waves of the workgroup, DEPTH block tiles in flight per wave.
template <typename QT, int D, int DEPTH>
__device__ __forceinline__ void prefix_item(const PrefixParams& p, int item) {
  typedef Mfma<QT> M;
  constexpr int NC = D / 32, NN = D / 16;
  constexpr int ROW_BYTES = 2 * D;
  constexpr int LANES_PER_ROW = ROW_BYTES / 16;
  constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;
  constexpr int VCH = kBS / ROWS_PER_PASS;
  constexpr int VROW = 2 * D + 16;   // LDS bytes per staged V row (padded)
  constexpr float kSlack = 8.0f;     // rescale only when a score passes the max by 2^8
  constexpr int RS = D + 4;          // floats per state row in LDS

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kvh = item % p.num_kv_heads;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int nrows = p.num_seqs * G;
  const int r0 = (item / p.num_kv_heads) * kPrefixRows;
  const int g = lane & 15;    // column of S^T / out^T
  const int kg = lane >> 4;   // lane group: k-chunk of the operands, 4-row slab of the outputs
  uint8_t* vst = lds + wave * kBS * VROW;
  int* tab = reinterpret_cast<int*>(lds + kPrefixWaves * kBS * VROW);
  float* states = reinterpret_cast<float*>(tab + kPrefixTable);
  // query / record row of row r
  auto qrow = [&](int r) { return (size_t)(r / G) * p.num_q_heads + kvh * G + r % G; };

  // the B operands: column g of group cg is row r0 + 16 cg + g (zeros past the last row)
  typename M::vec8 qop[kPrefixCG][NC];
#pragma unroll
  for (int cg = 0; cg < kPrefixCG; ++cg) {
    const int r = r0 + 16 * cg + g;
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p.query) + qrow(r < nrows ? r : 0) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 v = r < nrows ? *reinterpret_cast<const uint4*>(q + 32 * c + 8 * kg) : make_uint4(0, 0, 0, 0);
      qop[cg][c] = __builtin_bit_cast(typename M::vec8, v);
    }
  }
  float m2[kPrefixCG], lsum[kPrefixCG];
  floatx4 acc[kPrefixCG][NN];
#pragma unroll
  for (int cg = 0; cg < kPrefixCG; ++cg) {
    m2[cg] = -INFINITY;
    lsum[cg] = 0.f;
#pragma unroll
    for (int n = 0; n < NN; ++n) acc[cg][n] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int row_stride = p.num_kv_heads * ROW_BYTES;   // bytes between token rows
  const int tile_bytes = (kBS - 1) * row_stride + ROW_BYTES;
  const uint8_t* k_head = reinterpret_cast<const uint8_t*>(p.k_cache) + (size_t)kvh * ROW_BYTES;
  const uint8_t* v_head = reinterpret_cast<const uint8_t*>(p.v_cache) + (size_t)kvh * ROW_BYTES;
  // K: lane (row g, group kg) reads elements 32c + 8kg .. +7 of its row, the
  // A operand of MFMA c; V: whole rows, LANES_PER_ROW lanes per row
  const int k_off = g * row_stride + 16 * kg;
  int v_off[VCH], v_row[VCH];
#pragma unroll
  for (int ps = 0; ps < VCH; ++ps) {
    v_row[ps] = ps * ROWS_PER_PASS + lane / LANES_PER_ROW;
    v_off[ps] = v_row[ps] * row_stride + (lane % LANES_PER_ROW) * 16;
  }

  struct Tile {
    uint4 k[NC];
    uint4 v[VCH];
  };
  // entry j of the staged table; j >= end reads nothing (zero-size resource)
  auto load_tile = [&](Tile& t, int j, int end) {
    const bool valid = j < end;
    const int pb = __builtin_amdgcn_readfirstlane(tab[valid ? j : 0]);
    const size_t tile = (size_t)pb * kBS * row_stride;
    const int nbytes = valid ? tile_bytes : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k_head + tile, nbytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v_head + tile, nbytes);
#pragma unroll
    for (int c = 0; c < NC; ++c) t.k[c] = buf_load16(kr, k_off + 64 * c);
#pragma unroll
    for (int ps = 0; ps < VCH; ++ps) t.v[ps] = buf_load16(vr, v_off[ps]);
  };

  auto process = [&](const Tile& t) {
#pragma unroll
    for (int ps = 0; ps < VCH; ++ps)
      *reinterpret_cast<uint4*>(vst + v_row[ps] * VROW + (lane % LANES_PER_ROW) * 16) = t.v[ps];
    shortx4 pop[kPrefixCG];
#pragma unroll
    for (int cg = 0; cg < kPrefixCG; ++cg) {
      floatx4 sacc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc = M::qk(__builtin_bit_cast(typename M::vec8, t.k[c]), qop[cg][c], sacc);
      // lane holds tokens 4 kg + i of the block for column g
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = sacc[i] * p.scale_log2;
      const float lm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      if (__ballot(lm > m2[cg] + kSlack)) {
        float bmax = fmaxf(lm, __shfl_xor(lm, 16, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        const float mnew = fmaxf(m2[cg], bmax);
        const float alpha = __builtin_amdgcn_exp2f(m2[cg] - mnew);   // 0 while m2 = -inf
        lsum[cg] *= alpha;
#pragma unroll
        for (int n = 0; n < NN; ++n) acc[cg][n] *= alpha;
        m2[cg] = mnew;
      }
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(sc[i] - m2[cg]);
      const uint32_t p01 = M::pack2(pr[0], pr[1]);
      const uint32_t p23 = M::pack2(pr[2], pr[3]);
      // the denominator sums the 16-bit weights the MFMA uses
      lsum[cg] = M::acc2(p23, M::acc2(p01, lsum[cg]));
      pop[cg] = __builtin_bit_cast(shortx4, make_uint2(p01, p23));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane i of each 16-lane group reads row 4kg + i/4, columns 4(i%4)..+3
    const uint8_t* rd = vst + (4 * kg + (g >> 2)) * VROW + (g & 3) * 8;
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      const shortx4 vt = M::tr_read(rd + n * 32);
#pragma unroll
      for (int cg = 0; cg < kPrefixCG; ++cg) acc[cg][n] = M::pv(vt, pop[cg], acc[cg][n]);
    }
  };

  const int P = p.num_prefix_blocks;
  for (int c0 = 0; c0 < P; c0 += kPrefixTable) {
    const int cn = min(kPrefixTable, P - c0);
    __syncthreads();   // the previous chunk's entries are no longer read
    for (int i = threadIdx.x; i < cn; i += 64 * kPrefixWaves) {
      const int pb = p.table[c0 + i];
      tab[i] = (pb < 0 || pb >= p.num_blocks) ? 0 : pb;   // a bad table must not leave the caches
    }
    __syncthreads();
    // this wave's blocks: entries [j0, j1) of the chunk
    const int j0 = wave * cn / kPrefixWaves, j1 = (wave + 1) * cn / kPrefixWaves;
    const int n = j1 - j0;
    Tile ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_tile(ring[d], j0 + d, j1);
    __builtin_amdgcn_sched_barrier(0);
    for (int k0 = 0; k0 < n; k0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int k = k0 + d;
        if (k < n) process(ring[d]);
        __builtin_amdgcn_sched_barrier(0);
        load_tile(ring[d], j0 + k + DEPTH, j1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // the waves' states -> LDS, then one record per row
#pragma unroll
  for (int cg = 0; cg < kPrefixCG; ++cg) {
    float l = lsum[cg] + __shfl_xor(lsum[cg], 16, 64);
    l += __shfl_xor(l, 32, 64);
    float* st = states + (size_t)(wave * kPrefixRows + 16 * cg + g) * RS;
#pragma unroll
    for (int n = 0; n < NN; ++n) *reinterpret_cast<floatx4*>(st + 16 * n + 4 * kg) = acc[cg][n];
    if (kg == 0) {
      st[D] = m2[cg];
      st[D + 1] = l;
    }
  }
  __syncthreads();
  // thread -> (row rr, eighth ch of its D elements), 32 rows per pass; a
  // wave that took no block has m = -inf and weighs nothing
  const int ch = threadIdx.x & 7;
  for (int rr = threadIdx.x >> 3; rr < kPrefixRows; rr += 64 * kPrefixWaves / 8) {
    const int r = r0 + rr;
    if (r >= nrows) break;
    float mw[kPrefixWaves], mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kPrefixWaves; ++w) {
      mw[w] = states[(w * kPrefixRows + rr) * RS + D];
      mx = fmaxf(mx, mw[w]);
    }
    float wt[kPrefixWaves], l = 0.f;
#pragma unroll
    for (int w = 0; w < kPrefixWaves; ++w) {
      wt[w] = __builtin_amdgcn_exp2f(mw[w] - mx);
      l += wt[w] * states[(w * kPrefixRows + rr) * RS + D + 1];
    }
    float* dst = p.rec + qrow(r) * RS;
    constexpr int E = D / 8;   // elements per thread
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      floatx4 a = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kPrefixWaves; ++w)
        a += wt[w] * *reinterpret_cast<const floatx4*>(states + (w * kPrefixRows + rr) * RS + ch * E + e);
      *reinterpret_cast<floatx4*>(dst + ch * E + e) = a;
    }
    if (ch == 0) *reinterpret_cast<floatx4*>(dst + D) = floatx4{mx, l, 0.f, 0.f};
  }
}

template <typename QT, int D>
__global__ __launch_bounds__(64 * kPrefixWaves) void prefix_attn_kernel(PrefixParams p) {
  prefix_item<QT, D, 2>(p, blockIdx.x);
}

template <typename QT, int D>
static int launch_prefix_d(const PrefixParams& p, hipStream_t st) {
  auto kernel = prefix_attn_kernel<QT, D>;
  static std::atomic<bool> lds_set[64];
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(kernel), prefix_lds_bytes<D>(), lds_set);
  if (e != hipSuccess) return e;
  const int G = p.num_q_heads / p.num_kv_heads;
  const dim3 grid(((p.num_seqs * G + kPrefixRows - 1) / kPrefixRows) * p.num_kv_heads);
  kernel<<<grid, 64 * kPrefixWaves, prefix_lds_bytes<D>(), st>>>(p);
  return hipGetLastError();
}

int prefix_item_count(int num_seqs, int num_q_heads, int num_kv_heads) {
  const long long rows = (long long)num_seqs * (num_q_heads / num_kv_heads);
  return (int)((rows + kPrefixRows - 1) / kPrefixRows) * num_kv_heads;
}

int prefix_workgroups(int num_seqs, int num_q_heads, int num_kv_heads, int cus) {
  // the prefix role needs four waves per workgroup
  const int per_group = wave_group_size(num_kv_heads);
  if (per_group < kPrefixWaves) return 0;
  const int groups = (num_kv_heads + per_group - 1) / per_group;
  const int items = prefix_item_count(num_seqs, num_q_heads, num_kv_heads);
  // one item per workgroup, at most one per compute unit
  const int along_x = (items + groups - 1) / groups;
  return along_x * groups <= cus ? along_x : 0;
}

int launch_prefix_attn(const void* query, int q_dtype, const void* k_cache, const void* v_cache,
                       const int32_t* table, int prefix_blocks, float* records, int num_seqs, int num_q_heads,
                       int num_kv_heads, int head_dim, int num_blocks, float sm_scale, void* stream) {
  if (num_seqs == 0 || prefix_blocks == 0) return hipSuccess;
  PrefixParams p;
  p.query = query;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.table = table;
  p.rec = records;
  p.num_prefix_blocks = prefix_blocks;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.num_blocks = num_blocks;
  p.scale_log2 = sm_scale * kLog2e;
  p.items = prefix_item_count(num_seqs, num_q_heads, num_kv_heads);
  hipStream_t st = (hipStream_t)stream;
  if (q_dtype == PKV_BF16) return head_dim == 64 ? launch_prefix_d<BF16, 64>(p, st) : launch_prefix_d<BF16, 128>(p, st);
  return head_dim == 64 ? launch_prefix_d<F16, 64>(p, st) : launch_prefix_d<F16, 128>(p, st);
}

// ===========================================================================
// launchers
// ===========================================================================
static AttnParams make_params(const AttnArgs& a) {
  AttnParams p;
  p.out = a.out;
  p.query = a.query;
  p.k_cache = a.k_cache;
  p.v_cache = a.v_cache;
  p.k_scales = a.k_scales;
  p.v_scales = a.v_scales;
  p.block_tables = a.block_tables;
  p.seq_lens = a.seq_lens;
  p.ws = a.ws;
  p.plan = a.plan;
  p.rec_floats = (int)partial_record_floats(a.num_q_heads / a.num_kv_heads * (a.qtok > 0 ? a.qtok : 1), a.head_dim);
  p.num_seqs = a.num_seqs;
  // a selected decode takes lengths as they are (its pages come with the selection)
  p.mbs = a.selected ? (1 << 27) - 1 : a.max_blocks_per_seq;
  p.tstride = a.table_stride > 0 ? a.table_stride : p.mbs;
  p.len_off = a.len_off;
  p.srec = a.srec;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.num_blocks = a.num_blocks;
  p.partition_size = a.partition_size;
  p.num_partitions = a.num_partitions;
  p.sink = a.sink_tokens;
  p.window = a.window_tokens;
  p.min_units = a.min_units;
  p.list_cap = a.list_cap;
  p.selected = a.selected;
  p.budget = a.budget;
  p.qtok = a.qtok > 0 ? a.qtok : 1;
  p.table_bytes = a.selected ? (int)((long long)a.num_seqs * a.num_kv_heads * a.budget * 8)
                             : (int)(((long long)(a.num_seqs - 1) * p.tstride + a.max_blocks_per_seq) * 4);
  p.k_chan = a.k_chan;
  p.new_k = a.new_k;
  p.new_v = a.new_v;
  p.positions = a.positions;
  p.slots_out = a.slots_out;
  p.scale_log2 = a.sm_scale * kLog2e;
  p.pfx_wgs = 0;
  p.pfx = PrefixParams{};
  return p;
}

template <typename QT, typename KVT, int D, bool STREAM, bool SEL, bool GRP = false>
static int launch_wave(const AttnParams& p, int num_slots, hipStream_t st) {
  // (workgroup slot, group of up to 8 KV heads); one wave per KV head
  const int per_group = wave_group_size(p.num_kv_heads);
  const int groups = (p.num_kv_heads + per_group - 1) / per_group;
  const int lds = wave_group_lds(WaveCfg<KVT, D, GRP>::VSTAGE, per_group, p.list_cap);
  auto kernel = paged_attn_wave_kernel<QT, KVT, D, STREAM, SEL, GRP>;
  // above the default dynamic-LDS limit: the largest group needs ~105 KB
  static std::atomic<bool> lds_set[64];
  const int most = wave_group_lds(WaveCfg<KVT, D, GRP>::VSTAGE, kMaxWavesPerGroup, 128 * kMaxWavesPerGroup);
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(kernel), most, lds_set);
  if (e != hipSuccess) return e;
  kernel<<<dim3(num_slots, groups), 64 * per_group, lds, st>>>(p);
  return hipGetLastError();
}

template <typename QT, typename KVT>
static int launch_wave_d(const AttnParams& p, int num_slots, int D, bool stream, hipStream_t st) {
  // a selected decode reads scattered pages with the default load policy
  if (p.selected)
    return D == 64 ? launch_wave<QT, KVT, 64, false, true>(p, num_slots, st)
                   : launch_wave<QT, KVT, 128, false, true>(p, num_slots, st);
  if (stream)
    return D == 64 ? launch_wave<QT, KVT, 64, true, false>(p, num_slots, st)
                   : launch_wave<QT, KVT, 128, true, false>(p, num_slots, st);
  return D == 64 ? launch_wave<QT, KVT, 64, false, false>(p, num_slots, st)
                 : launch_wave<QT, KVT, 128, false, false>(p, num_slots, st);
}

// INT4 caches: head_dim 128 only (a lane group's quarter row is one 16-byte load)
template <typename QT>
static int launch_wave_i4(const AttnParams& p, int num_slots, bool stream, hipStream_t st) {
  if (p.selected) return launch_wave<QT, I4, 128, false, true>(p, num_slots, st);
  if (stream) return launch_wave<QT, I4, 128, true, false>(p, num_slots, st);
  return launch_wave<QT, I4, 128, false, false>(p, num_slots, st);
}

template <typename QT, typename KVT, int D>
static int launch_simple(const AttnParams& p, dim3 grid, hipStream_t st) {
  paged_attn_simple_kernel<QT, KVT, D><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

// Grouped scales: INT8 (head_dim 64 or 128) and INT4 (head_dim 128) codes.
template <typename QT>
static int launch_wave_grouped(const AttnParams& p, int num_slots, int kv_dtype, int D, bool stream,
                               hipStream_t st) {
  if (kv_dtype == PKV_I4)
    return stream ? launch_wave<QT, I4, 128, true, false, true>(p, num_slots, st)
                  : launch_wave<QT, I4, 128, false, false, true>(p, num_slots, st);
  if (D == 64)
    return stream ? launch_wave<QT, I8, 64, true, false, true>(p, num_slots, st)
                  : launch_wave<QT, I8, 64, false, false, true>(p, num_slots, st);
  return stream ? launch_wave<QT, I8, 128, true, false, true>(p, num_slots, st)
                : launch_wave<QT, I8, 128, false, false, true>(p, num_slots, st);
}

int launch_paged_attn_partition(const AttnArgs& a) {
  if (a.num_seqs == 0) return hipSuccess;
  AttnParams p = make_params(a);
  if (a.k_chan) {
    const bool stream = (a.flags & PKV_DECODE_STREAM_KV) != 0;
    return a.q_dtype == PKV_BF16
               ? launch_wave_grouped<BF16>(p, a.num_slots, a.kv_dtype, a.head_dim, stream, (hipStream_t)a.stream)
               : launch_wave_grouped<F16>(p, a.num_slots, a.kv_dtype, a.head_dim, stream, (hipStream_t)a.stream);
  }
  hipStream_t st = (hipStream_t)a.stream;
  const int D = a.head_dim;
  if (a.kv_dtype == PKV_F32) {
    const dim3 grid(a.num_kv_heads, a.num_partitions, a.num_seqs);
    return D == 64 ? launch_simple<F32, F32, 64>(p, grid, st) : launch_simple<F32, F32, 128>(p, grid, st);
  }
  const int K = a.num_slots;
  const bool stream = (a.flags & PKV_DECODE_STREAM_KV) != 0;
  if (a.q_dtype == PKV_BF16) {
    switch (a.kv_dtype) {
      case PKV_BF16: return launch_wave_d<BF16, BF16>(p, K, D, stream, st);
      case PKV_I8: return launch_wave_d<BF16, I8>(p, K, D, stream, st);
      case PKV_I4: return launch_wave_i4<BF16>(p, K, stream, st);
      case PKV_FP8E5M2: return launch_wave_d<BF16, BF8>(p, K, D, stream, st);
      default: return launch_wave_d<BF16, FP8>(p, K, D, stream, st);
    }
  }
  switch (a.kv_dtype) {
    case PKV_F16: return launch_wave_d<F16, F16>(p, K, D, stream, st);
    case PKV_I8: return launch_wave_d<F16, I8>(p, K, D, stream, st);
    case PKV_I4: return launch_wave_i4<F16>(p, K, stream, st);
    case PKV_FP8E5M2: return launch_wave_d<F16, BF8>(p, K, D, stream, st);
    default: return launch_wave_d<F16, FP8>(p, K, D, stream, st);
  }
}

// The combined shared-prefix launch (16-bit caches of the query's type):
// pfx_wgs workgroups along x of prefix items, then the decode's slots.
template <typename QT, int D, bool STREAM>
static int launch_wave_pfx(const AttnParams& p, int num_slots, hipStream_t st) {
  const int per_group = wave_group_size(p.num_kv_heads);
  const int groups = (p.num_kv_heads + per_group - 1) / per_group;
  const int wave_lds = wave_group_lds(WaveCfg<QT, D>::VSTAGE, per_group, p.list_cap);
  const int lds = wave_lds > prefix_lds_bytes<D>() ? wave_lds : prefix_lds_bytes<D>();
  auto kernel = paged_attn_wave_kernel<QT, QT, D, STREAM, false, false, true>;
  static std::atomic<bool> lds_set[64];
  const int wmost = wave_group_lds(WaveCfg<QT, D>::VSTAGE, kMaxWavesPerGroup, 128 * kMaxWavesPerGroup);
  const int most = wmost > prefix_lds_bytes<D>() ? wmost : prefix_lds_bytes<D>();
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(kernel), most, lds_set);
  if (e != hipSuccess) return e;
  kernel<<<dim3(p.pfx_wgs + num_slots, groups), 64 * per_group, lds, st>>>(p);
  return hipGetLastError();
}

int launch_shared_prefix_decode(const AttnArgs& a, const int32_t* prefix_table, int prefix_blocks, float* prefix_rec,
                                int pfx_wgs) {
  if (a.num_seqs == 0) return hipSuccess;
  AttnParams p = make_params(a);
  p.pfx_wgs = pfx_wgs;
  p.pfx.query = a.query;
  p.pfx.k_cache = a.k_cache;
  p.pfx.v_cache = a.v_cache;
  p.pfx.table = prefix_table;
  p.pfx.rec = prefix_rec;
  p.pfx.num_prefix_blocks = prefix_blocks;
  p.pfx.num_seqs = a.num_seqs;
  p.pfx.num_q_heads = a.num_q_heads;
  p.pfx.num_kv_heads = a.num_kv_heads;
  p.pfx.num_blocks = a.num_blocks;
  p.pfx.scale_log2 = a.sm_scale * kLog2e;
  p.pfx.items = prefix_item_count(a.num_seqs, a.num_q_heads, a.num_kv_heads);
  hipStream_t st = (hipStream_t)a.stream;
  const bool stream = (a.flags & PKV_DECODE_STREAM_KV) != 0;
  const int K = a.num_slots;
  if (a.q_dtype == PKV_BF16) {
    if (a.head_dim == 64) return stream ? launch_wave_pfx<BF16, 64, true>(p, K, st) : launch_wave_pfx<BF16, 64, false>(p, K, st);
    return stream ? launch_wave_pfx<BF16, 128, true>(p, K, st) : launch_wave_pfx<BF16, 128, false>(p, K, st);
  }
  if (a.head_dim == 64) return stream ? launch_wave_pfx<F16, 64, true>(p, K, st) : launch_wave_pfx<F16, 64, false>(p, K, st);
  return stream ? launch_wave_pfx<F16, 128, true>(p, K, st) : launch_wave_pfx<F16, 128, false>(p, K, st);
}

int launch_paged_attn_merge(const AttnArgs& a) {
  if (a.num_seqs == 0) return hipSuccess;
  const int T = a.qtok > 0 ? a.qtok : 1;
  const dim3 grid(a.num_q_heads * T, a.num_seqs);
  hipStream_t st = (hipStream_t)a.stream;
  const int rec = (int)partial_record_floats(a.num_q_heads / a.num_kv_heads * T, a.head_dim);
  if (a.q_dtype == PKV_F32) {
    if (a.num_partitions <= 1) return hipSuccess;
    const int max_len = a.max_blocks_per_seq * a.block_size;
    if (a.head_dim == 64)
      paged_attn_merge_units_kernel<F32, 64><<<grid, 256, 0, st>>>(a.out, a.seq_lens, a.ws, rec, a.num_q_heads,
                                                                    a.num_kv_heads, a.num_partitions,
                                                                    a.partition_size, max_len);
    else
      paged_attn_merge_units_kernel<F32, 128><<<grid, 256, 0, st>>>(a.out, a.seq_lens, a.ws, rec, a.num_q_heads,
                                                                     a.num_kv_heads, a.num_partitions,
                                                                     a.partition_size, max_len);
    return hipGetLastError();
  }
  if (!a.may_split && !a.srec) return hipSuccess;
  // columns per workgroup: halved from a whole record row (at most 256
  // threads' worth of 16-byte pieces) while the grid is under ~1024
  // workgroups
  const int NCOL = a.num_q_heads / a.num_kv_heads * T;
  int cpw = NCOL < 1024 / a.head_dim ? NCOL : 1024 / a.head_dim;
  const long long pairs = (long long)a.num_seqs * a.num_kv_heads;
  while (cpw > 1 && pairs * ((NCOL + cpw - 1) / cpw) < 1024) cpw = (cpw + 1) / 2;
  const dim3 mgrid(a.num_seqs, a.num_kv_heads, (NCOL + cpw - 1) / cpw);
#define PKV_MERGE(QT, D)                                                                                   \
  paged_attn_merge_kernel<QT, D><<<mgrid, 256, 0, st>>>(a.out, a.ws, a.plan, rec, a.num_q_heads, a.num_kv_heads, \
                                                        T, cpw, a.prefix, a.srec)
  if (a.head_dim == 64) {
    if (a.q_dtype == PKV_BF16) PKV_MERGE(BF16, 64);
    else PKV_MERGE(F16, 64);
  } else {
    if (a.q_dtype == PKV_BF16) PKV_MERGE(BF16, 128);
    else PKV_MERGE(F16, 128);
  }
#undef PKV_MERGE
  return hipGetLastError();
}

}  // namespace pkv
