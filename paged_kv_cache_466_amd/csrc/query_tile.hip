// Query-tile pass for gfx950: many query tokens of one sequence against its
// paged cache (a chunk of prefill, or a speculative batch longer than the
// decode's 16 MFMA columns per KV head), read block by block through the
// sequence's block table ("Chapter 18", "How PagedAttention Works"; the
// Learning-AI topic t13_4 block table), GQA as in "KV Cache Engineering"
// section 1.  Launched by pkv_paged_attn_decode_multi when the query rows per
// KV head exceed 16.
#include <hip/hip_runtime.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {
constexpr int kBS = 16;                     // tokens per block
constexpr float kLog2e = 1.4426950408889634f;
}  // namespace

// ===========================================================================
// Query-tile pass: many query tokens of one sequence (a chunk of prefill)
//
// With T new tokens per sequence whose keys and values are already in the
// cache at positions L - T .. L - 1, token t attends to positions
// 0 .. L - T + t (the causal reading of several new tokens; the pages stop
// at one token per step).  For one (sequence, KV head) the T * G query rows
// (row r is token r / G, head r % G of the group) against the sequence's
// blocks are a dense product, Q [T G, D] x K^T [D, L], followed by P.V: the
// matrix cores' work.
//
// A workgroup of NW waves takes 32 * NW rows of one (sequence, KV head); each
// wave owns 32 of them (two 16-row column groups) outright.  The workgroup
// walks the blocks some row of the tile can see through a ring of NBUF block
// slots in LDS: each block's K and V tiles are loaded once for all waves,
// straight from memory into LDS (buffer loads with the LDS destination),
// each wave fetching its share of the tile's 1 KB pieces.  A tile's 16-byte
// chunk c of row r sits at position c ^ (r mod chunks-per-row) of its LDS
// row, so that the key reads of the q.K operand (16 rows, one chunk) and the
// transposing reads of V (4 rows, 32 bytes each, per 16 lanes) spread over
// the banks.  V rows at or past L load with an out-of-range offset, which
// writes zeros: the unwritten slots of a last block may hold anything.
// Per block a wave computes S^T = K Q^T for both column groups
// (v_mfma_f32_16x16x32, the key operand read from LDS) and out^T += V^T P^T
// for both from one transposed read of V (v_mfma_f32_16x16x16), with a
// causal limit per row in the blocks past its first row's.  One barrier per
// block: after it, the block is complete in LDS and every wave is done with
// the slot the next load overwrites.  Rows leave normalised, staged through
// LDS as whole-line stores.
// ===========================================================================
// s_waitcnt immediate: vmcnt(n) (bits 3:0 and 15:14), lgkmcnt(0), expcnt left alone
constexpr int waitcnt_vmcnt(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | 0x0070; }

constexpr int kChunkCG = 2;                 // 16-row column groups per wave
constexpr int kChunkWaveRows = 16 * kChunkCG;
constexpr int kChunkNBuf = 6;               // block slots in the LDS ring (three pairs)
constexpr int kChunkTable = 1024;           // table entries staged in LDS at a time


struct ChunkParams {
  void* out;              // [S][T][Hq][D]
  const void* query;      // [S][T][Hq][D]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  int mbs, num_seqs, qtok, num_q_heads, num_kv_heads, num_blocks;
  float scale_log2;
};

// Three waves per SIMD for the 4-wave workgroups (160 VGPRs at head_dim 128).
// The 2-wave ones need a few registers more and run at two; a 1-wave
// workgroup's LDS ring leaves room for at most one wave per SIMD.
template <typename QT, int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW >= 4 ? 3 : NW))) void chunk_attn_kernel(
    ChunkParams p) {
  typedef Mfma<QT> M;
  constexpr int NC = D / 32, NN = D / 16;
  constexpr int ROWB = 2 * D;              // bytes of one token row of one head
  constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  constexpr int TILE = kBS * ROWB;         // one K or V tile
  constexpr int SLOT = 2 * TILE;
  constexpr int PIECES = 2 * TILE / 1024;  // 1 KB pieces (one wave-wide load each) of a block
  static_assert(PIECES % NW == 0, "every wave loads the same number of pieces");
  constexpr int LPW = PIECES / NW;         // loads per wave per block
  constexpr float kSlack = 8.0f;           // rescale only when a score passes the max by 2^8
  constexpr int RS = D + 4;                // floats per staged output row

  // The ring's slots are separate LDS objects, and the block loop is unrolled
  // so that each step names the slot it reads and the slot it loads into:
  // the compiler then knows that the reads do not touch what the loads in
  // flight write, and waits for the loads only where this code does.
  static_assert(kChunkNBuf == 6, "six ring slots");
  __shared__ __attribute__((aligned(16))) uint8_t ring0[SLOT], ring1[SLOT], ring2[SLOT], ring3[SLOT], ring4[SLOT],
      ring5[SLOT];
  __shared__ int tab[kChunkTable];
  auto ring = [&](int i) -> uint8_t* {
    return i == 0 ? ring0 : i == 1 ? ring1 : i == 2 ? ring2 : i == 3 ? ring3 : i == 4 ? ring4 : ring5;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = p.num_q_heads / p.num_kv_heads;
  const int T = p.qtok;
  const int nrows = T * G;
  // Workgroup n runs on XCD n % 8.  The row tiles of one (sequence, KV
  // head) read the same blocks, so they all go to one XCD, whose L2 then
  // serves the tiles after the first: pair xcd + 8 (j / R), tile j % R for
  // the j-th workgroup of XCD xcd (R tiles per pair; the grid is padded to
  // whole groups of 8 pairs).
  const int R = (nrows + 32 * NW - 1) / (32 * NW);
  const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3;
  const int pair = xcd + 8 * (jw / R);
  if (pair >= p.num_seqs * p.num_kv_heads) return;
  const int s = pair / p.num_kv_heads, kvh = pair % p.num_kv_heads;
  const int r0 = (jw % R) * 32 * NW;          // the workgroup's first row
  const int w0 = r0 + wave * kChunkWaveRows;  // this wave's first row
  const int g = lane & 15;    // column of S^T / out^T
  const int kg = lane >> 4;   // lane group: k-chunk of the operands, 4-row slab of the outputs
  // query / output element offset of row r
  auto qrow = [&](int r) {
    const int t = r / G;
    return (((size_t)s * T + t) * p.num_q_heads + kvh * G + (r - t * G)) * D;
  };

  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.mbs * kBS ? p.mbs * kBS : L);
  // token t sees positions 0 .. L - T + t: the workgroup's rows up to
  // lim_hi, all of this wave's up to wlim_lo
  const int lim_hi = L - T + min(r0 + 32 * NW - 1, nrows - 1) / G;
  const int wlim_lo = L - T + min(w0, nrows - 1) / G;
  const int nvis = lim_hi < 0 ? 0 : min((L + kBS - 1) / kBS, lim_hi / kBS + 1);
  const bool has_rows = w0 < nrows;

  // the B operands: column g of group cg is row w0 + 16 cg + g (zeros past the last row)
  typename M::vec8 qop[kChunkCG][NC];
  int lim[kChunkCG];
#pragma unroll
  for (int cg = 0; cg < kChunkCG; ++cg) {
    const int r = w0 + 16 * cg + g;
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p.query) + qrow(r < nrows ? r : 0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 v = r < nrows ? *reinterpret_cast<const uint4*>(q + 32 * c + 8 * kg) : make_uint4(0, 0, 0, 0);
      qop[cg][c] = __builtin_bit_cast(typename M::vec8, v);
    }
    lim[cg] = L - T + (r < nrows ? r : nrows - 1) / G;
  }
  float m2[kChunkCG], lsum[kChunkCG];
  floatx4 acc[kChunkCG][NN];
#pragma unroll
  for (int cg = 0; cg < kChunkCG; ++cg) {
    m2[cg] = -INFINITY;
    lsum[cg] = 0.f;
#pragma unroll
    for (int n = 0; n < NN; ++n) acc[cg][n] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int row_stride = p.num_kv_heads * ROWB;   // bytes between token rows
  const int tile_bytes = (kBS - 1) * row_stride + ROWB;
  const uint8_t* k_head = reinterpret_cast<const uint8_t*>(p.k_cache) + (size_t)kvh * ROWB;
  const uint8_t* v_head = reinterpret_cast<const uint8_t*>(p.v_cache) + (size_t)kvh * ROWB;
  // this lane's chunk of each piece it loads: LDS chunk q = 64 * piece + lane
  // of the tile is row q / CPR, position q % CPR, which holds the row's chunk
  // (q % CPR) ^ (row % CPR)
  int ld_row[LPW], ld_off[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int piece = (wave * LPW + u) % (PIECES / 2);
    const int q = 64 * piece + lane;
    ld_row[u] = q / CPR;
    ld_off[u] = ld_row[u] * row_stride + (((q % CPR) ^ (ld_row[u] % CPR)) * 16);
  }
  // block j of the staged table chunk (logical block c0 + j) into slot
  // `slot`; j >= cn loads nothing (zero-size resource)
  auto issue = [&](uint8_t* slot, int j, int cn, int c0) {
    const bool valid = j < cn;
    const int pb = __builtin_amdgcn_readfirstlane(tab[valid ? j : 0]);
    const size_t tile = (size_t)pb * kBS * row_stride;
    const int nbytes = valid ? tile_bytes : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k_head + tile, nbytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v_head + tile, nbytes);
    const int t0 = (c0 + j) * kBS;
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int pc = wave * LPW + u;            // piece of the block: K pieces, then V pieces
      const bool isv = pc >= PIECES / 2;
      const int piece = isv ? pc - PIECES / 2 : pc;
      uint8_t* dst = slot + (isv ? TILE : 0) + piece * 1024;
      const int off = isv && t0 + ld_row[u] >= L ? kOutOfRange : ld_off[u];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? vr : kr, (__attribute__((address_space(3))) void*)dst, 16, off,
                                               0, 0, 0);
    }
  };

  // per-lane LDS offsets of the operand reads (swizzled chunk positions)
  int k_rd[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) k_rd[c] = g * ROWB + (((4 * c + kg) ^ (g % CPR)) * 16);
  const int vr_row = 4 * kg + (g >> 2);
  int v_rd[NN];
#pragma unroll
  for (int n = 0; n < NN; ++n)
    v_rd[n] = TILE + vr_row * ROWB + (((2 * n + ((g & 3) >> 1)) ^ (vr_row % CPR)) * 16) + (g & 1) * 8;

  // Two blocks a, b (tokens t0 .. t0 + 31) per step: one softmax update per
  // 32 tokens, and P.V over both blocks as one v_mfma_f32_16x16x32 per 16
  // channels.  Its k index 8 kg + i is token 4 kg + i of block a for i < 4
  // and of block b for i >= 4: the score tiles of a and b give P^T in that
  // order, and the transposed reads of a's and b's V give V^T in it.
  auto process2 = [&](const uint8_t* sa, const uint8_t* sb, int t0) {
    // some position of a block lies past some of this wave's rows' limits
    const bool msk_a = t0 + kBS - 1 > wlim_lo, msk_b = t0 + 2 * kBS - 1 > wlim_lo;
    floatx4 sacc[2][kChunkCG];
#pragma unroll
    for (int cg = 0; cg < kChunkCG; ++cg) sacc[0][cg] = sacc[1][cg] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 ka = *reinterpret_cast<const uint4*>(sa + k_rd[c]);
      const uint4 kb = *reinterpret_cast<const uint4*>(sb + k_rd[c]);
#pragma unroll
      for (int cg = 0; cg < kChunkCG; ++cg) {
        sacc[0][cg] = M::qk(__builtin_bit_cast(typename M::vec8, ka), qop[cg][c], sacc[0][cg]);
        sacc[1][cg] = M::qk(__builtin_bit_cast(typename M::vec8, kb), qop[cg][c], sacc[1][cg]);
      }
    }
    // lane holds tokens 4 kg + i of each block for column g; raw scores, the
    // factor is applied inside the exponent (positive, so maxima commute)
    float lm[kChunkCG];
#pragma unroll
    for (int cg = 0; cg < kChunkCG; ++cg) {
      if (msk_a) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 4 * kg + i > lim[cg]) sacc[0][cg][i] = -INFINITY;
      }
      if (msk_b) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + kBS + 4 * kg + i > lim[cg]) sacc[1][cg][i] = -INFINITY;
      }
      const float ma = fmaxf(fmaxf(sacc[0][cg][0], sacc[0][cg][1]), fmaxf(sacc[0][cg][2], sacc[0][cg][3]));
      const float mbk = fmaxf(fmaxf(sacc[1][cg][0], sacc[1][cg][1]), fmaxf(sacc[1][cg][2], sacc[1][cg][3]));
      lm[cg] = fmaxf(ma, mbk) * p.scale_log2;
    }
    typename M::vec8 pop[kChunkCG];
#pragma unroll
    for (int cg = 0; cg < kChunkCG; ++cg) {
      // a row that has seen no visible position yet and sees none here keeps
      // alpha = 1 and weights 0 (exp2(-inf - -inf) would be NaN)
      if (__ballot(lm[cg] > m2[cg] + kSlack)) {
        float bmax = fmaxf(lm[cg], __shfl_xor(lm[cg], 16, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        const float mnew = fmaxf(m2[cg], bmax);
        const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m2[cg] - mnew);
        lsum[cg] *= alpha;
#pragma unroll
        for (int n = 0; n < NN; ++n) acc[cg][n] *= alpha;
        m2[cg] = mnew;
      }
      const float mb = (msk_b & (m2[cg] == -INFINITY)) ? 0.f : m2[cg];
      float pr[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(fmaf(sacc[0][cg][i], p.scale_log2, -mb));
        pr[4 + i] = __builtin_amdgcn_exp2f(fmaf(sacc[1][cg][i], p.scale_log2, -mb));
      }
      const uint4 pw = make_uint4(M::pack2(pr[0], pr[1]), M::pack2(pr[2], pr[3]), M::pack2(pr[4], pr[5]),
                                  M::pack2(pr[6], pr[7]));
      // the denominator sums the 16-bit weights the MFMA uses
      lsum[cg] = M::acc2(pw.w, M::acc2(pw.z, M::acc2(pw.y, M::acc2(pw.x, lsum[cg]))));
      pop[cg] = __builtin_bit_cast(typename M::vec8, pw);
    }
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      const shortx4 va = M::tr_read(sa + v_rd[n]);
      const shortx4 vb = M::tr_read(sb + v_rd[n]);
      const typename M::vec8 vt = __builtin_bit_cast(
          typename M::vec8, make_uint4(__builtin_bit_cast(uint2, va).x, __builtin_bit_cast(uint2, va).y,
                                       __builtin_bit_cast(uint2, vb).x, __builtin_bit_cast(uint2, vb).y));
#pragma unroll
      for (int cg = 0; cg < kChunkCG; ++cg) acc[cg][n] = M::qk(vt, pop[cg], acc[cg][n]);
    }
  };

  for (int c0 = 0; c0 < nvis; c0 += kChunkTable) {
    const int cn = min(kChunkTable, nvis - c0);
    __syncthreads();   // every wave is done with the ring and the previous entries
    const int32_t* trow = p.block_tables + (size_t)s * p.mbs + c0;
    for (int i = threadIdx.x; i < cn; i += 64 * NW) {
      const int pb = trow[i];
      tab[i] = (pb < 0 || pb >= p.num_blocks) ? 0 : pb;   // a bad table must not leave the caches
    }
    __syncthreads();
    // The ring holds three pairs of blocks; block b sits in slot b mod 6.
    // Step k waits for its own pair (pair k + 1 may still be in flight),
    // then, after the barrier (every wave's pieces have landed and every wave
    // is done with pair k - 1), loads pair k + 2 into the slots pair k - 1
    // used and works on pair k.  Past the end the loads are zero-size: the
    // rows of such a block read as zeros and its scores are masked (its
    // positions lie past every row's limit).
    issue(ring0, 0, cn, c0);
    issue(ring1, 1, cn, c0);
    issue(ring2, 2, cn, c0);
    issue(ring3, 3, cn, c0);
    for (int j = 0; j < cn; j += 6) {
#pragma unroll
      for (int h = 0; h < 3; ++h) {
        const int jj = j + 2 * h;
        // A plain s_barrier: __syncthreads()'s release fence would also wait
        // for the loads of the next pair, which this step does not need.  The
        // clobber keeps the compiler from moving memory accesses across it.
        __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(2 * LPW));
        asm volatile("s_barrier" ::: "memory");
        issue(ring((2 * h + 4) % 6), jj + 4, cn, c0);
        issue(ring((2 * h + 5) % 6), jj + 5, cn, c0);
        if (has_rows && jj < cn) process2(ring(2 * h), ring(2 * h + 1), (c0 + jj) * kBS);
      }
    }
  }
  // the last issued pieces (zero-size, past the chunk) land before the ring
  // is reused for the output rows
  __builtin_amdgcn_s_waitcnt(0x0070);
  __syncthreads();
  if (!has_rows) return;

  // ---- normalised rows through this wave's share of the ring -------------
  float inv[kChunkCG];
#pragma unroll
  for (int cg = 0; cg < kChunkCG; ++cg) {
    float l = lsum[cg] + __shfl_xor(lsum[cg], 16, 64);
    l += __shfl_xor(l, 32, 64);
    inv[cg] = l > 0.f ? 1.f / l : 0.f;
  }
  float* st = reinterpret_cast<float*>(ring(wave));
  static_assert(8 * RS * 4 <= SLOT, "eight staged rows fit a ring slot");
  constexpr int CPO = D / 8;   // 16-byte pieces of an output row
#pragma unroll
  for (int q = 0; q < 4; ++q) {   // rows 8q .. 8q + 7 of the wave's 32
    const int cg = q >> 1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if ((g >> 3) == (q & 1)) {
#pragma unroll
      for (int n = 0; n < NN; ++n)
        *reinterpret_cast<floatx4*>(st + (g & 7) * RS + 16 * n + 4 * kg) = acc[cg][n] * inv[cg];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int rbase = w0 + 8 * q;
    const int rows = min(8, nrows - rbase);
    for (int c = lane; c < rows * CPO; c += 64) {
      const float* src = st + (c / CPO) * RS + (c % CPO) * 8;
      const floatx4 lo = *reinterpret_cast<const floatx4*>(src);
      const floatx4 hi = *reinterpret_cast<const floatx4*>(src + 4);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + qrow(rbase + c / CPO) + (c % CPO) * 8) =
          make_uint4(M::pack2(lo[0], lo[1]), M::pack2(lo[2], lo[3]), M::pack2(hi[0], hi[1]), M::pack2(hi[2], hi[3]));
    }
  }
}

template <typename QT, int D, int NW>
static int launch_chunk_nw(const ChunkParams& p, hipStream_t st) {
  auto kernel = chunk_attn_kernel<QT, D, NW>;
  const int G = p.num_q_heads / p.num_kv_heads;
  const long long tiles = (p.qtok * G + 32 * NW - 1) / (32 * NW);
  const long long pairs8 = ((long long)p.num_seqs * p.num_kv_heads + 7) / 8 * 8;
  kernel<<<dim3((unsigned)(pairs8 * tiles)), 64 * NW, 0, st>>>(p);
  return hipGetLastError();
}

// waves per workgroup: enough for the rows (32 each), at most 4
template <typename QT, int D>
static int launch_chunk_d(const ChunkParams& p, hipStream_t st) {
  const int rows = p.qtok * (p.num_q_heads / p.num_kv_heads);
  if (rows <= 32) return launch_chunk_nw<QT, D, 1>(p, st);
  if (rows <= 64) return launch_chunk_nw<QT, D, 2>(p, st);
  return launch_chunk_nw<QT, D, 4>(p, st);
}

int launch_chunk_attn(const AttnArgs& a) {
  if (a.num_seqs == 0) return hipSuccess;
  ChunkParams p;
  p.out = a.out;
  p.query = a.query;
  p.k_cache = a.k_cache;
  p.v_cache = a.v_cache;
  p.block_tables = a.block_tables;
  p.seq_lens = a.seq_lens;
  p.mbs = a.max_blocks_per_seq;
  p.num_seqs = a.num_seqs;
  p.qtok = a.qtok;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.num_blocks = a.num_blocks;
  p.scale_log2 = a.sm_scale * kLog2e;
  hipStream_t st = (hipStream_t)a.stream;
  if (a.q_dtype == PKV_BF16) return a.head_dim == 64 ? launch_chunk_d<BF16, 64>(p, st) : launch_chunk_d<BF16, 128>(p, st);
  return a.head_dim == 64 ? launch_chunk_d<F16, 64>(p, st) : launch_chunk_d<F16, 128>(p, st);
}

}  // namespace pkv
