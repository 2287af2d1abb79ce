// Paged decode attention for CDNA4 (gfx950).
//
// What is computed: for each sequence, one new query token per query head
// attends over the sequence's cached K/V. The cache sits in physical blocks
// of 8, 16 or 32 tokens that the sequence's block table maps from logical
// blocks ("vLLM:
// Anatomy and Mechanisms of High-Throughput LLM Inference", section
// "Block-Level Management"; decode semantics from "Inside vLLM: Anatomy of a
// High-Throughput LLM Inference System", section "Scheduler").
//
// Work split (balanced). KV heads form groups of HG heads (HG = largest
// divisor of num_kv_heads that is <= 4). A "unit" is one 16-token chunk of
// one sequence for one head group (a block with 16-token blocks, half a
// 32-token block, two 8-token blocks); a "segment" is all units of one
// (sequence, head group), in logical order. Segments are laid end to end in
// (sequence, head group) order, and workgroup w takes units
// [w*U/E, (w+1)*U/E) of the U in total, E = min(W, U) of the W workgroups
// (the last W - E get nothing), whatever the context lengths are, so
// every workgroup moves the same number of K/V bytes and the grid has no long
// tail. A workgroup has one wavefront per KV head of the group; all of its
// wavefronts walk the same blocks, so the 2 KiB token rows of a group are read
// together. Each workgroup finds its start itself: it sums and scans the
// clamped context lengths (cheap next to the K/V it streams).
//
// A segment that lies inside one workgroup is finished there and written as
// bf16. A segment cut by workgroup boundaries leaves fp32 partials (running
// max in base 2, sum, unnormalised output) from each piece; the workgroup
// that holds its last unit records which pieces exist, and merge_kernel
// combines them with log-sum-exp weights after the decode kernel.
//
// Inner loop, per chunk (16 tokens), on matrix cores:
//   * QK^T on v_mfma_f32_16x16x32_bf16: rows are the 16 tokens of the block,
//     columns the 16 query-head slots, the reduction runs over head_size.
//     Lane (c, grp) (c = lane % 16, grp = lane / 16) loads, for MFMA step j,
//     the 16 bytes at head dims 32*j + 8*grp of token c's row; q is loaded
//     with the same mapping (the sum over head_size is order-free). The
//     result gives lane (c, grp) the logits of query head c for tokens
//     4*grp .. 4*grp+3.
//   * V is transposed (tokens along registers) by an MFMA with a one-hot
//     16x16 selector (v_mfma_f32_16x16x16_bf16): lane (c, grp) receives
//     V[4*grp + r][d(c)], r = 0..3, exactly the tokens whose probabilities it
//     holds. The values are exact bf16, so their upper halves repack into an
//     operand with v_perm.
//   * P*V on v_mfma_f32_16x16x16_bf16 with P split into two bf16 terms (high
//     part plus rounding residue), which keeps about 16 significant bits of
//     P. The accumulators leave lane (c, grp) with output dims
//     32*j + 8*grp .. +7 of query head c, stored as 16-byte vectors.
// Online softmax works in base 2 (logits prescaled by scale*log2 e, hardware
// exp2). Row maxima are shared by the four lanes of a head with two
// cross-lane exchanges per block; row sums stay lane-partial until the end.
//
// Tokens past the context length are never fetched (the last block's buffer
// range ends at the context length, so those rows read as zeros), their
// logits are masked by a select and their V rows are zeroed again, so stale
// data in the tail of the last block (even NaN) cannot reach the output. Block ids are clamped to the pool, and no
// table entry past a sequence's last used block is read.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// The unit of work is a chunk of 16 tokens (one MFMA tile of rows): with
// 16-token cache blocks a chunk is a block, a 32-token block holds two
// chunks, and a chunk holds two 8-token blocks.
constexpr int kBlock = 16;

template <int BS>
constexpr int chunk_of() { return kBlock; }
constexpr uint32_t kBf16One = 0x3F80u;

// What a decode launch computes: one new token per sequence (kSingle);
// several, each with its own causal limit (kCausal); the same with more than
// 32 (new token, query head) columns per KV head (kWide: a workgroup's
// wavefronts are the column groups of one KV head, 32 columns each); or a
// list of items, each read once for the one or more sequences it serves
// (kShared); or one new token per sequence that is not in the cache yet
// (kStep): it is read from the step's new K/V rows as one more chunk at the
// end of its sequence, and written to its slot in the same launch.
constexpr int kSingle = 0, kCausal = 1, kShared = 2, kWide = 3, kStep = 4;

// Chunks of a segment of n positions: the cached ones in CH-token chunks,
// and (kStep) the newest position on its own as the last chunk.
template <int M, int CH>
__device__ __forceinline__ int seg_chunks(int n) {
  if constexpr (M == kStep) return n > 0 ? (n - 1 + CH - 1) / CH + 1 : 0;
  return (n + CH - 1) / CH;
}

// Several new tokens per sequence, each with its own causal limit.
constexpr bool causal(int M) { return M == kCausal || M == kWide; }

__device__ __forceinline__ f32x4_t mfma32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16(u32x2_t a, u32x2_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                   __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// Upper halves of two fp32 words that hold exact bf16 values: lo | hi << 16.
__device__ __forceinline__ uint32_t pack_hi(float lo, float hi) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo),
                               0x07060302u);
}

// Two fp32 values rounded to bf16 (nearest even): lo | hi << 16.
__device__ __forceinline__ uint32_t to_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4_t load16(const uint16_t *p) {
  return *reinterpret_cast<const u32x4_t *>(p);
}

__device__ __forceinline__ int clamp_len(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }

// The two values of lanes i and i ^ 16 (lane_pair16) or i and i ^ 32
// (lane_pair32), lower lane first, by the gfx950 lane-swap instructions
// (vector ALU; no LDS round trip). Both lanes of a pair get the same two
// values in the same order, so a max or a sum of them is the same in both.
// The instruction swaps rows between two registers that both hold x; it is
// written as an asm statement (a register-only ALU instruction, preceded by
// the two wait states a lane swap needs after a vector write of its
// sources). Through the compiler builtin, hipcc (gfx950) treated the two
// results as one value and dropped the max of them.
__device__ __forceinline__ void lane_pair16(float x, float &lo, float &hi) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = a;
  hi = b;
}
__device__ __forceinline__ void lane_pair32(float x, float &lo, float &hi) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = a;
  hi = b;
}

// Max and sum over the four lanes c, c + 16, c + 32, c + 48 (the four
// lane groups of a 16-wide MFMA column or of a token's head dims).
__device__ __forceinline__ float max_over_groups(float x) {
  float a, b;
  lane_pair16(x, a, b);
  lane_pair32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_over_groups(float x) {
  float a, b;
  lane_pair16(x, a, b);
  lane_pair32(a + b, a, b);
  return a + b;
}

// Workgroup w's first unit, w <= E: floor(w * U / E). With E <= U every
// range is non-empty.
__device__ __forceinline__ long long range_lo(long long w, long long U, long long E) {
  return w * U / E;
}

// The workgroup whose range holds unit u: the w with lo(w) <= u < lo(w+1).
__device__ __forceinline__ int owner_of(long long u, long long U, long long E) {
  return (int)(((u + 1) * E - 1) / U);
}

// Store the lane's outputs as bf16: accumulator tiles 2j and 2j+1 hold head
// dims 32*j + 8*grp + 0..3 and + 4..7; `dst` already points at 8*grp.
template <int NJ>
__device__ __forceinline__ void store_out(uint16_t *dst, const f32x4_t (&acc)[2 * NJ], float inv) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const f32x4_t a = acc[2 * j] * inv;
    const f32x4_t b = acc[2 * j + 1] * inv;
    u32x4_t w = {to_bf16x2(a[0], a[1]), to_bf16x2(a[2], a[3]), to_bf16x2(b[0], b[1]),
                 to_bf16x2(b[2], b[3])};
    *reinterpret_cast<u32x4_t *>(dst + 32 * j) = w;
  }
}

// Sum of `v` over the workgroup (every thread gets the result). `red` holds
// one slot per wavefront; the call starts and ends with a barrier so it can
// be called repeatedly.
__device__ __forceinline__ long long wg_sum(long long v, long long *red, int wave, int lane,
                                            int nwaves) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  long long t = 0;
  for (int i = 0; i < nwaves; ++i) t += red[i];
  return t;
}

// Inclusive prefix sum of `v` over the workgroup's threads in thread order.
// Also returns the sum over the lower-numbered wavefronts (`pre`, to add to
// the result) and over the whole workgroup (`total`). Starts and ends with a
// barrier so it can be called repeatedly.
__device__ __forceinline__ long long wg_scan(long long v, long long *red, int wave, int lane, int nwaves,
                                             long long &pre, long long &total) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  __syncthreads();
  if (lane == 63) red[wave] = v;
  __syncthreads();
  pre = 0;
  total = 0;
  for (int i = 0; i < nwaves; ++i) {
    if (i < wave) pre += red[i];
    total += red[i];
  }
  return v;
}

// A piece is the run of blocks of one (sequence, head group) that lies in
// this workgroup's range of units.
struct Piece {
  long long seg_start;  // first unit of the segment the piece belongs to
  int s;                // sequence (an item, in kShared)
  int hg;               // head group
  int off;              // first block of the piece, counted from the segment's first
  int cnt;              // blocks in the piece (>= 1)
  int n;                // positions < n are visible (the clamped context length)
  int L;                // blocks of the segment
  bool first;           // the workgroup's first piece
  // kShared only: the item's table row, first q row, q rows, first own
  // chunk and shared cache blocks (otherwise row s is read from block 0
  // with q_len q rows).
  int row, qrow, ntok, b0, eb;
};

// Produces the workgroup's pieces in order. Every thread of the workgroup
// runs the same walk; the state is uniform, and so are the addresses of the
// context lengths it reads (scalar loads).
struct Walker {
  const int32_t *lens;
  const ShareItem *items;
  int S, NG, cap;  // S: sequences, or items in kShared
  int S_rows;      // kShared: the batch's sequences (q and output rows)
  long long u, hi, seg_base;
  int s, hg, off, L, n;
  int row, qrow, ntok, b0, eb;
  bool first;
};

// The item's fields are uniform; readfirstlane keeps them in scalar
// registers (the buffer ranges and table reads built from them must be).
// The rows an item names are clamped to the batch (num_seqs = wk.S_rows),
// so a plan made for other sizes gives wrong results, never an access
// outside q, the tables or the output.
__device__ __forceinline__ void take_item(Walker &wk, const ShareItem &x) {
  const int S = wk.S_rows;
  wk.eb = __builtin_amdgcn_readfirstlane(x.eb);
  wk.L = __builtin_amdgcn_readfirstlane(x.L);
  wk.n = __builtin_amdgcn_readfirstlane(x.n);
  wk.row = min(max(__builtin_amdgcn_readfirstlane(x.row), 0), S - 1);
  wk.qrow = min(max(__builtin_amdgcn_readfirstlane(x.qrow), 0), S - 1);
  wk.ntok = min(max(__builtin_amdgcn_readfirstlane(x.ntok), 1), S - wk.qrow);
  wk.b0 = __builtin_amdgcn_readfirstlane(x.b0);
}

template <int M, int CH = kBlock>
__device__ __forceinline__ bool next_piece(Walker &wk, Piece &p) {
  if (wk.u >= wk.hi) return false;
  if constexpr (M == kShared) {
    p.row = wk.row;
    p.qrow = wk.qrow;
    p.ntok = wk.ntok;
    p.b0 = wk.b0;
    p.eb = wk.eb;
  }
  p.s = wk.s;
  p.hg = wk.hg;
  p.off = wk.off;
  p.n = wk.n;
  p.L = wk.L;
  p.cnt = (int)min((long long)(wk.L - wk.off), wk.hi - wk.u);
  p.seg_start = wk.seg_base + (long long)wk.hg * wk.L;
  p.first = wk.first;
  wk.first = false;
  wk.u += p.cnt;
  wk.off += p.cnt;
  if (wk.off == wk.L) {
    wk.off = 0;
    if (++wk.hg == wk.NG && wk.u < wk.hi) {
      wk.hg = 0;
      wk.seg_base += (long long)wk.NG * wk.L;
      do {  // units remain, so a non-empty sequence (item) follows
        ++wk.s;
        if constexpr (M == kShared) {
          if (wk.s < wk.S) take_item(wk, wk.items[wk.s]); else wk.L = 0;
        } else {
          wk.n = wk.s < wk.S ? clamp_len(wk.lens[wk.s], wk.cap) : 0;
          wk.L = seg_chunks<M, CH>(wk.n);
        }
      } while (wk.L == 0 && wk.s < wk.S);
      if (wk.s >= wk.S) wk.u = wk.hi;  // only if the lengths changed during the call
    }
  }
  return true;
}

// Per-thread constants of the decode kernel. A wavefront serves one KV head;
// its MFMA columns are (new token, query head) pairs of that head, token-
// major (column = token * group + head), 16 per tile. Lane (c, grp) holds
// column 16*t + c of tile t.
template <int NT>
struct Lane {
  int tid, wave, lane, c, grp, w;
  int HG, NG;
  bool col_ok[NT];       // the lane's column of tile t exists (column < q_len * group)
  int col[NT];           // that column, or the last one when it does not exist
  int lcol[NT];          // the same counted within the wavefront's column group (kWide; else = col)
  int qshift[NT];        // q_len - 1 - new token of the column: its causal limit is n - qshift
  int tok[NT];           // the column's new token (kShared: its member of the segment)
  uint32_t q_off[NT];    // byte offset of the lane's 16 bytes of its column's q row (in the
                         // sequence's q rows from the KV head's first query head on)
  uint32_t out_off[NT];  // element offset of the lane's 8 outputs, same origin
  size_t blk_stride;     // elements per block of one cache array
  int row_bytes;         // bytes per token row of one cache array (all KV heads)
  uint32_t lane_off;     // byte offset of the lane's 16 bytes in (block, head): token c, dims 8*grp..
  uint32_t lane_off_b;   // 8-token blocks: the same in the chunk's second block (rows 8-15), or 2 GiB
                         // (past any block's range) for rows 0-7
  long long U, E;
  uint32_t pool32;       // min(num_blocks, INT32_MAX)
  u32x2_t sel;
};

// The KV head a wavefront serves in head group hg: one head per wavefront,
// or (kWide) the group's one head for every wavefront.
template <int M, int NT>
__device__ __forceinline__ int kv_head(const Lane<NT> &ln, int hg) {
  return M == kWide ? hg : hg * ln.HG + ln.wave;
}

// kShared: one chunk of a segment's stream: read through member j's table
// row (or the segment's `row` for the first member's chunks before b0), and
// seen by members j .. e.
struct Cursor {
  int j;    // member reading the chunk
  int e;    // last member that sees it
  int b;    // chunk
  int n;    // member j's context length
  int row;  // table row read
};

// One wavefront's pass over its workgroup's stream of blocks.
template <int NJ, int NT>
struct Stream {
  Piece P, Q;            // the piece being computed and the next one
  bool has_q;
  int i;                 // block of P being computed
  int ord;               // P's position among the workgroup's pieces
  size_t hoff, hoff_q;
  u32x4_t qv[NT][NJ];    // q of P, in the MFMA operand layout (one column tile only)
  float m_run[NT];       // running max of base-2 logits, per column
  float l_part[NT];      // this lane's share of the running sum
  f32x4_t acc[NT][2 * NJ];
  // kShared: cursor of block i of P, and the member records of P's and Q's
  // segments (lane j: member j).
  Cursor cc;
  int2 mv_p, mv_q;
  // Launches that defer (defers()): the first piece's partial record when that piece is
  // cut, and the workgroup's merge record. Both are stored after the stream
  // ends, not when the first piece ends: the wait for every later block's
  // loads would otherwise also wait for those stores to complete.
  f32x4_t first_acc[2 * NJ];
  float first_m, first_l;
  bool first_cut;
  int2 desc;
  int staged;  // whole-segment outputs staged in LDS
  int nnew;    // kStep: new K/V rows staged in LDS for their slots
};

// Buffer-resource word 3 for gfx9-family raw (untyped) buffer loads.
constexpr int kRawBufferWord3 = 0x00020000;
// Cache-policy operand of a buffer load: the nt (non-temporal) bit.
constexpr int kNonTemporal = 2;

// bf16 outputs of whole segments are staged in LDS and stored after the
// stream (launches that defer, below), as many per wavefront as the launch
// leaves room for (stage_slots; more are stored at once). Stores issued
// mid-stream are counted with the loads in flight, so the wait for the next
// blocks would also wait for them to complete. With many short sequences a
// wavefront ends dozens of segments: 4096 sequences of median 64 tokens
// (32 segments per wavefront) measured 264.0 us with 16 outputs staged,
// 251.1 with 24 and 240.8 with 32 (two launches).
// Each wavefront may take this much LDS: a quarter of the compute unit's
// 160 KiB (four wavefronts, or four one-wavefront workgroups, per unit),
// less a margin for the kernel's static LDS.
constexpr int kLdsPerWave = 163840 / 4 - 256;
constexpr int kMaxStageSlots = 64;

// Whether the current piece's q stays in registers for the whole piece
// (one column tile; and sharing-aware decode with two tiles, where it fits
// in 218 VGPRs and measured 5% faster than reading q from LDS every block).
// Otherwise, with two tiles, q is parked in LDS at the piece switch.
template <int NT, int M, int BS>
constexpr bool q_in_regs() { return NT == 1 || (M == kShared && BS != 8); }

// Whether a launch defers those stores: one column tile, and not with
// 8-token blocks, whose loop measured 8% slower with the deferred state in
// registers (240 -> 260 us on the GQA layer).
template <int NT, int BS>
constexpr bool defers() { return NT == 1 && BS != 8; }

// q rows of the piece's columns for this wavefront, in the MFMA operand
// layout. Read through a buffer resource (scalar base at the KV head's first
// query head of the sequence's first new token, fixed lane offsets) so that
// no vector address is computed here.
template <int NJ, int NT, int M>
__device__ __forceinline__ void load_q(const DecodeArgs &a, const Lane<NT> &ln, const Piece &p,
                                       u32x4_t (&qv)[NT][NJ]) {
  constexpr int D = NJ * 32;
  // q rows of the piece: its sequence's q_len rows, or an item's ntok rows
  // (columns past them read as zeros and are never stored).
  const size_t row0 = M == kShared ? (size_t)p.qrow : (size_t)p.s * a.q_len;
  const int rows = M == kShared ? p.ntok : a.q_len;
  const size_t base = (row0 * a.num_q_heads + (size_t)kv_head<M>(ln, p.hg) * a.group) * D * sizeof(uint16_t);
  const int span = ((rows - 1) * a.num_q_heads + a.group) * D * (int)sizeof(uint16_t);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(reinterpret_cast<const char *>(a.q) + base), 0, span, kRawBufferWord3);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      qv[t][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, ln.q_off[t] + 64 * j, 0, 0));
}

// A q row in LDS: head_size bf16 values and 16 bytes of padding. Lanes
// c = 0..15 of a 16-byte read take the rows of 16 columns at the same head
// dims; with rows 256 bytes apart (head_size 128) all 16 would fall in the
// same banks, and the read would take 16 passes instead of 4 (measured: LDS
// bank conflicts 41% of the compute units' cycles with 64 new tokens).
template <int NJ>
constexpr int q_row() { return NJ * 32 + 8; }

// q of the next piece travels through LDS (one column tile only): two slots
// per wavefront, each holding the KV head's column rows [num_cols][q_row]
// as bf16; slot = piece position & 1.
template <int NJ>
__device__ __forceinline__ uint16_t *q_slot(uint16_t *lds, const DecodeArgs &a, int wave, int ord) {
  return lds + ((size_t)wave * 2 + (ord & 1)) * a.num_cols * q_row<NJ>();
}

// Launches that defer: the wavefront's output staging area (after the q ring of
// every wavefront): stage_slots bf16 outputs, then their row offsets padded
// to 16 bytes (stage_stride bytes in all). An output occupies num_cols * D
// bf16 values, lane (c, grp) holding 8 consecutive values for each MFMA step
// j at ((j * 4 + grp) * num_cols + c) * 8.
__host__ __device__ __forceinline__ int stage_out_bytes(int slots, int num_cols, int D) {
  return slots * num_cols * D * (int)sizeof(uint16_t);
}
__host__ __device__ __forceinline__ int stage_stride(int slots, int num_cols, int D) {
  return stage_out_bytes(slots, num_cols, D) + (slots * (int)sizeof(size_t) + 15) / 16 * 16;
}
template <int NJ>
__device__ __forceinline__ uint16_t *stage_area(uint16_t *lds, const DecodeArgs &a, int wave) {
  return lds + (size_t)a.heads_per_wg * 2 * a.num_cols * q_row<NJ>() +
         (size_t)wave * stage_stride(a.stage_slots, a.num_cols, NJ * 32) / sizeof(uint16_t);
}
template <int NJ>
__device__ __forceinline__ size_t *stage_dsts(uint16_t *area, const DecodeArgs &a) {
  return reinterpret_cast<size_t *>(area + stage_out_bytes(a.stage_slots, a.num_cols, NJ * 32) / sizeof(uint16_t));
}

// kStep: the new K/V rows a wavefront writes to their slots are staged here
// and stored after the stream, up to kNewSlots per wavefront (more are
// stored at once). A slot holds the K row, the V row (head_size bf16 each)
// and the destination element offset, padded to 16 bytes.
constexpr int kNewSlots = 24;
template <int D>
constexpr int new_slot_elems() { return 2 * D + 8; }

template <int NJ>
__device__ __forceinline__ uint16_t *new_area(uint16_t *lds, const DecodeArgs &a, int wave) {
  constexpr int D = NJ * 32;
  return lds + (size_t)a.heads_per_wg * 2 * a.num_cols * q_row<NJ>() +
         (size_t)a.heads_per_wg * stage_stride(a.stage_slots, a.num_cols, D) / sizeof(uint16_t) +
         (size_t)wave * kNewSlots * new_slot_elems<D>();
}

template <int NJ>
__device__ __forceinline__ int stage_slots(const DecodeArgs &a) {
  return a.stage_slots;
}

// The one slot per wavefront that holds the current piece's q (two tiles):
// [rec_cols][q_row], the wavefront's own columns.
template <int NJ>
__device__ __forceinline__ uint16_t *q_park(uint16_t *lds, const DecodeArgs &a, int wave) {
  return lds + (size_t)wave * a.rec_cols * q_row<NJ>();
}

// With two column tiles the current piece's q lives in LDS (one slot per
// wavefront, [num_cols][q_row]), loaded at the piece switch and read per block:
// the registers to keep it, or to stage the next piece's, are not there.
// Each lane writes and reads only its own columns' rows (or, for a missing
// column, the last row, written by the same wavefront), so no barrier is
// needed.
template <int NJ, int NT>
__device__ __forceinline__ void park_q(uint16_t *slot, const Lane<NT> &ln, const u32x4_t (&qv)[NT][NJ]) {
  uint16_t *qs = slot + ln.grp * 8;
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (ln.col_ok[t]) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) *reinterpret_cast<u32x4_t *>(qs + ln.lcol[t] * q_row<NJ>() + 32 * j) = qv[t][j];
    }
}

template <int NJ, int NT>
__device__ __forceinline__ void parked_q(const uint16_t *slot, const Lane<NT> &ln, int t, u32x4_t (&qv)[NJ]) {
  const uint16_t *qs = slot + ln.lcol[t] * q_row<NJ>() + ln.grp * 8;
#pragma unroll
  for (int j = 0; j < NJ; ++j) qv[j] = *reinterpret_cast<const u32x4_t *>(qs + 32 * j);
}

// Physical block of logical block b of sequence s, clamped to the pool. The
// address is uniform, so this is a scalar load: waiting for it never waits
// for the K/V loads in flight.
// pool32 = min(num_blocks, INT32_MAX): one unsigned compare, in scalar
// registers, rejects negative ids and ids past the pool.
__device__ __forceinline__ int block_id(const int32_t *__restrict__ tables, const DecodeArgs &a, uint32_t pool32,
                                        int s, int b) {
  const int id = tables[(size_t)s * a.max_blocks_per_seq + b];
  return (uint32_t)id < pool32 ? id : 0;
}

// kShared: the plan's records of a segment's members, lane j holding member
// j's: its context length (x) and the chunks before its own (y), those it
// holds in common with member j - 1. Lanes past the last member read {0, 0}.
// y is clamped to the member's chunks, so no count below goes negative.
__device__ __forceinline__ int2 member_info(const int32_t *__restrict__ members, const Piece &p, int lane, int cap) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t *>(members + 2 * (size_t)p.qrow), 0, p.ntok * 2 * (int)sizeof(int32_t), kRawBufferWord3);
  const int n = clamp_len((int)__builtin_amdgcn_raw_buffer_load_b32(r, lane * 8, 0, 0), cap);
  const int y = (int)__builtin_amdgcn_raw_buffer_load_b32(r, lane * 8 + 4, 0, 0);
  return int2{n, min(max(y, 0), (n + kBlock - 1) >> 4)};
}

// kShared: the cursor of member j's chunk b. The members after j that hold
// it are those up to the first whose own chunks begin at or before b (a
// ballot over the lanes of the members' records).
__device__ __forceinline__ Cursor seg_at(const Piece &p, int j, int b, int nj, int2 mv, int lane) {
  const unsigned long long stop = __builtin_amdgcn_ballot_w64(lane > j && lane < p.ntok && mv.y <= b);
  const int e = stop ? (int)__builtin_ctzll(stop) - 1 : p.ntok - 1;
  return Cursor{j, e, b, nj, b < p.b0 ? p.row : p.qrow + j};
}

// kShared: cursor of the segment's chunk at unit offset p.off (the piece's
// first). Member j contributes its chunks from y_j on.
__device__ __forceinline__ Cursor seg_first(const Piece &p, int2 mv, int lane) {
  int r = p.off;
  int j = 0, nj = 0, yj = 0;
  for (; j < p.ntok; ++j) {
    nj = __builtin_amdgcn_readlane(mv.x, j);
    yj = __builtin_amdgcn_readlane(mv.y, j);
    const int lj = ((nj + kBlock - 1) >> 4) - yj;
    if (r < lj) break;
    r -= lj;
  }
  if (j == p.ntok) --j;  // past the segment's end: not reached inside a piece
  return seg_at(p, j, yj + r, nj, mv, lane);
}

// kShared: cursor of the segment's chunk after c (the same member's next
// chunk, else the next member's first own chunk).
__device__ __forceinline__ Cursor seg_next(const Piece &p, const Cursor &c, int2 mv, int lane) {
  if (c.b + 1 < ((c.n + kBlock - 1) >> 4)) return seg_at(p, c.j, c.b + 1, c.n, mv, lane);
  for (int j = c.j + 1; j < p.ntok; ++j) {
    const int nj = __builtin_amdgcn_readlane(mv.x, j);
    const int yj = __builtin_amdgcn_readlane(mv.y, j);
    if (((nj + kBlock - 1) >> 4) > yj) return seg_at(p, j, yj, nj, mv, lane);
  }
  return c;  // past the segment's end: not reached inside a piece
}

// Element offset of the wavefront's KV head inside a token row (uniform).
template <int NJ, int M, int NT>
__device__ __forceinline__ size_t head_off(const Lane<NT> &ln, const Piece &p) {
  return (size_t)kv_head<M>(ln, p.hg) * (NJ * 32);
}

// Starts the loads of one block's K and V rows for this wavefront's head.
// Each array is read through a buffer resource whose base is the (block,
// head) start (scalar registers) and whose size covers the block's first
// `nrows` token rows; the lane adds its fixed offset. So no vector address
// arithmetic happens per block, and the rows past the context length in a
// sequence's last block are never fetched: they read as zeros.
//
// Cache policy: the loads of the first half of each K row (at D = 128 its
// first 128-byte line) carry policy PK, the non-temporal hint unless several
// wavefronts read the same block, and every other load is plain, so about a
// quarter of the K/V bytes stream with the hint. Measured on
// MI355X against all-plain loads, this is 5-10% faster on every cold workload
// (e.g. the GQA layer 208 us against 226 us), and faster than hinting all of
// K (213 us) or all of K and V (225 us). Where the calls re-read blocks
// (beams sharing a prompt) it is also faster than all-plain (179 against
// 186 us).
template <int NJ, int NT, int PK = kNonTemporal>
__device__ __forceinline__ void issue_rows(const char *kb, const char *vb, const Lane<NT> &ln, int nrows,
                                           u32x4_t (&K)[NJ], u32x4_t (&V)[NJ]) {
  const int span = nrows * ln.row_bytes;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kb), 0, span, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vb), 0, span, kRawBufferWord3);
#pragma unroll
  for (int j = 0; j < NJ / 2; ++j)
    K[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, ln.lane_off + 64 * j, 0, PK));
#pragma unroll
  for (int j = NJ / 2; j < NJ; ++j)
    K[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, ln.lane_off + 64 * j, 0, 0));
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    V[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, ln.lane_off + 64 * j, 0, 0));
}

// The same for the first `nrows` token rows of block `blk` of the cache, at
// the wavefront's KV head (element offset hoff in a token row).
template <int NJ, int NT, int PK = kNonTemporal>
__device__ __forceinline__ void issue(const DecodeArgs &a, const Lane<NT> &ln, int blk, size_t hoff, int nrows,
                                      u32x4_t (&K)[NJ], u32x4_t (&V)[NJ]) {
  const size_t base = ((size_t)blk * ln.blk_stride + hoff) * sizeof(uint16_t);
  issue_rows<NJ, NT, PK>(reinterpret_cast<const char *>(a.k_cache) + base, reinterpret_cast<const char *>(a.v_cache) + base,
                 ln, nrows, K, V);
}

// Two 8-token blocks as one chunk: rows 0-7 of the tile from block `ida`
// (its first `na` rows), rows 8-15 from block `idb` (its first `nb`). Each
// lane loads from both blocks' resources: at its offset in the first block
// (past that block's range for rows 8-15) and at lane_off_b in the second
// (its row less 8, or 2 GiB for rows 0-7, past any range). The load outside
// its range reads as zero, so OR-ing the two gives the row without a
// per-lane choice of resource.
template <int NJ, int NT, int PK = kNonTemporal>
__device__ __forceinline__ void issue_pair_rows(const char *kba, const char *vba, int na, const char *kbb,
                                                const char *vbb, int nb, const Lane<NT> &ln, u32x4_t (&K)[NJ],
                                                u32x4_t (&V)[NJ]) {
  const __amdgpu_buffer_rsrc_t rka =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kba), 0, na * ln.row_bytes, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rkb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kbb), 0, nb * ln.row_bytes, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rva =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vba), 0, na * ln.row_bytes, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rvb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vbb), 0, nb * ln.row_bytes, kRawBufferWord3);
  const uint32_t off_b = ln.lane_off_b;
#pragma unroll
  for (int j = 0; j < NJ / 2; ++j)
    K[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rka, ln.lane_off + 64 * j, 0, PK)) |
           __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rkb, off_b + 64 * j, 0, PK));
#pragma unroll
  for (int j = NJ / 2; j < NJ; ++j)
    K[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rka, ln.lane_off + 64 * j, 0, 0)) |
           __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rkb, off_b + 64 * j, 0, 0));
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    V[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rva, ln.lane_off + 64 * j, 0, 0)) |
           __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rvb, off_b + 64 * j, 0, 0));
}

template <int NJ, int NT, int PK = kNonTemporal>
__device__ __forceinline__ void issue_pair(const DecodeArgs &a, const Lane<NT> &ln, int ida, int idb, size_t hoff,
                                           int na, int nb, u32x4_t (&K)[NJ], u32x4_t (&V)[NJ]) {
  const size_t base_a = ((size_t)ida * ln.blk_stride + hoff) * sizeof(uint16_t);
  const size_t base_b = ((size_t)idb * ln.blk_stride + hoff) * sizeof(uint16_t);
  const char *kc = reinterpret_cast<const char *>(a.k_cache), *vc = reinterpret_cast<const char *>(a.v_cache);
  issue_pair_rows<NJ, NT, PK>(kc + base_a, vc + base_a, na, kc + base_b, vc + base_b, nb, ln, K, V);
}

// kStep with 16- or 32-token blocks: the newest position of sequence s as a
// chunk of its own, read from the step's new K/V rows ([num_seqs,
// num_kv_heads, head_size]): it is row 0 of the tile; rows 1-15 lie past the
// one-row range and read as zeros. (With 8-token blocks issue_seq builds the
// same chunk in the two-block form.)
template <int NJ, int NT>
__device__ __forceinline__ void issue_new(const DecodeArgs &a, const Lane<NT> &ln, int s, size_t hoff,
                                          u32x4_t (&K)[NJ], u32x4_t (&V)[NJ]) {
  const size_t base = ((size_t)s * a.num_kv_heads * (NJ * 32) + hoff) * sizeof(uint16_t);
  issue_rows<NJ>(reinterpret_cast<const char *>(a.k_new) + base, reinterpret_cast<const char *>(a.v_new) + base, ln,
                 1, K, V);
}

// Starts the loads of chunk c of table row `row` for this wavefront's head,
// in a cache of BS-token blocks: block c (BS = 16), half of block c/2
// (BS = 32), or blocks 2c and 2c+1 (BS = 8; the second only if the chunk
// reaches into it).
template <int NJ, int NT, int BS, int PK = kNonTemporal>
__device__ __forceinline__ void issue_chunk(const int32_t *__restrict__ tables, const DecodeArgs &a,
                                            const Lane<NT> &ln, int row, int c, size_t hoff, int nrows,
                                            u32x4_t (&K)[NJ], u32x4_t (&V)[NJ]) {
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size 8, 16 or 32");
  if constexpr (BS < kBlock) {
    const int na = nrows < BS ? nrows : BS;
    const int nb = nrows - na;
    const int ida = block_id(tables, a, ln.pool32, row, 2 * c);
    const int idb = nb > 0 ? block_id(tables, a, ln.pool32, row, 2 * c + 1) : 0;
    issue_pair<NJ, NT, PK>(a, ln, ida, idb, hoff, na, nb, K, V);
  } else if constexpr (BS == kBlock) {
    issue<NJ, NT, PK>(a, ln, block_id(tables, a, ln.pool32, row, c), hoff, nrows, K, V);
  } else {
    issue<NJ, NT, PK>(a, ln, block_id(tables, a, ln.pool32, row, c >> 1),
              hoff + (size_t)(c & 1) * kBlock * (ln.row_bytes / sizeof(uint16_t)), nrows, K, V);
  }
}

// kShared: starts the loads of the segment's chunk at cursor c of piece p,
// through the cursor's table row, except that with 8-token blocks a chunk
// can begin with the last of the eb blocks a group shares (an odd count):
// that block comes through the segment's `row` too.
template <int NJ, int NT, int BS>
__device__ __forceinline__ void issue_shared(const int32_t *__restrict__ tables, const DecodeArgs &a,
                                             const Lane<NT> &ln, const Piece &p, const Cursor &c, size_t hoff,
                                             int nrows, u32x4_t (&K)[NJ], u32x4_t (&V)[NJ]) {
  if constexpr (BS < kBlock) {
    const int na = nrows < BS ? nrows : BS;
    const int nb = nrows - na;
    const int ida = block_id(tables, a, ln.pool32, 2 * c.b < p.eb ? p.row : c.row, 2 * c.b);
    const int idb = nb > 0 ? block_id(tables, a, ln.pool32, c.row, 2 * c.b + 1) : 0;
    issue_pair<NJ>(a, ln, ida, idb, hoff, na, nb, K, V);
  } else {
    issue_chunk<NJ, NT, BS>(tables, a, ln, c.row, c.b, hoff, nrows, K, V);
  }
}

// Token rows of chunk b (CH tokens) that lie before the context length n.
template <int CH = kBlock>
__device__ __forceinline__ int rows_in(int n, int b) {
  const int r = n - b * CH;
  return r < CH ? r : CH;
}

// Starts the loads of chunk b of sequence s (n positions, L chunks): from
// the cache, or (kStep) for the last chunk the step's new K/V row; the
// cached chunks of kStep end before the newest position.
template <int NJ, int NT, int M, int BS>
__device__ __forceinline__ void issue_seq(const int32_t *__restrict__ tables, const DecodeArgs &a, const Lane<NT> &ln,
                                          int s, int b, int n, int L, size_t hoff, u32x4_t (&K)[NJ],
                                          u32x4_t (&V)[NJ]) {
  constexpr int CH = chunk_of<BS>();
  if constexpr (M == kStep && BS < kBlock) {
    // One load sequence for both kinds of chunk. With a branch between the
    // two, the compiler completes each branch's OR of the two blocks' loads
    // before the join, which waits for the loads just issued and stalls the
    // pipeline (measured: 375 against 215 us on the GQA layer). The newest
    // position's chunk takes the first block's place with the new K/V row
    // and one row; the table is then read at entry 0, which every row has.
    const bool fresh = b == L - 1;
    const int nrows = fresh ? 1 : rows_in<CH>(n - 1, b);
    const int na = nrows < BS ? nrows : BS;
    const int nb = nrows - na;
    const int ida = block_id(tables, a, ln.pool32, s, fresh ? 0 : 2 * b);
    const int idb = nb > 0 ? block_id(tables, a, ln.pool32, s, 2 * b + 1) : 0;
    const char *kc = reinterpret_cast<const char *>(a.k_cache), *vc = reinterpret_cast<const char *>(a.v_cache);
    const size_t base_a = ((size_t)ida * ln.blk_stride + hoff) * sizeof(uint16_t);
    const size_t base_b = ((size_t)idb * ln.blk_stride + hoff) * sizeof(uint16_t);
    const size_t base_n = ((size_t)s * a.num_kv_heads * (NJ * 32) + hoff) * sizeof(uint16_t);
    const char *kba = fresh ? reinterpret_cast<const char *>(a.k_new) + base_n : kc + base_a;
    const char *vba = fresh ? reinterpret_cast<const char *>(a.v_new) + base_n : vc + base_a;
    issue_pair_rows<NJ>(kba, vba, na, kc + base_b, vc + base_b, nb, ln, K, V);
  } else if constexpr (M == kStep) {
    if (b == L - 1)
      issue_new<NJ>(a, ln, s, hoff, K, V);
    else
      issue_chunk<NJ, NT, BS>(tables, a, ln, s, b, hoff, rows_in<CH>(n - 1, b), K, V);
  } else {
    // Past 32 columns the wavefronts of a workgroup read the same blocks:
    // plain loads keep them in L2 for the others (64 new tokens: 1148
    // against 1192 us; 16: 430 against 474 us), where a single reader
    // streams faster with the hint on part of K.
    issue_chunk<NJ, NT, BS, M == kWide ? 0 : kNonTemporal>(tables, a, ln, s, b, hoff, rows_in<CH>(n, b), K, V);
  }
}

// Stores the partial record of column tile t of this wavefront in slot
// `slot` (0: the workgroup's first piece, 1: its last): unnormalised output,
// running max (base 2) and sum.
template <int NJ, int NT>
__device__ __forceinline__ void store_record(const DecodeArgs &a, const Lane<NT> &ln, int t, int slot,
                                             const f32x4_t (&acc)[2 * NJ], float m, float l) {
  constexpr int D = NJ * 32;
  const size_t row = (((size_t)ln.w * 2 + slot) * ln.HG + ln.wave) * a.rec_cols + ln.lcol[t];
  float *po = a.part_o + row * D + ln.grp * 8;
#pragma unroll
  for (int k = 0; k < 2 * NJ; ++k) *reinterpret_cast<f32x4_t *>(po + 32 * (k >> 1) + 4 * (k & 1)) = acc[k];
  if (ln.grp == 0) {
    if constexpr (NT == 1) {
      *reinterpret_cast<f32x2_t *>(a.part_ml + row * 2) = f32x2_t{m, l};
    } else {
      a.part_ml[row * 2] = m;
      a.part_ml[row * 2 + 1] = l;
    }
  }
}

// Writes P's result: bf16 output when P is a whole segment, otherwise its
// partial record. A workgroup's first piece is the only one that can end a
// segment begun in an earlier workgroup, so each workgroup writes one merge
// record, decided when its first piece ends: that segment and where its
// pieces are, or none. Launches that defer store the first piece's partial
// record, the merge record and staged outputs after the stream (finish_stream).
// DF: defer the first piece's record, the merge record and (up to the
// staging area's capacity) whole-segment outputs to finish_stream.
template <int NJ, int NT, int M, bool DF>
__device__ __forceinline__ void finish_piece(const DecodeArgs &a, const Lane<NT> &ln, Stream<NJ, NT> &st,
                                             uint16_t *lds) {
  constexpr int D = NJ * 32;
  constexpr bool kMulti = causal(M);
  const Piece &P = st.P;
  const bool whole = P.off == 0 && P.cnt == P.L;
  const int g = kv_head<M>(ln, P.hg);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float l = sum_over_groups(st.l_part[t]);
    // kShared: a segment serves ntok members (their q rows from qrow on).
    const bool keep = M == kShared ? ln.col_ok[t] && ln.col[t] < P.ntok * a.group : ln.col_ok[t];
    if (whole) {
      // With several new tokens a column can see no position at all (only
      // if a context is shorter than q_len), and so can an empty member of a
      // segment; it is written as zeros.
      const float inv = (kMulti || M == kShared) ? (l > 0.f ? 1.f / l : 0.f) : 1.f / l;
      const size_t row0 = M == kShared ? (size_t)P.qrow : (size_t)P.s * a.q_len;
      const size_t dst = (row0 * a.num_q_heads + (size_t)g * a.group) * D;
      if (DF && st.staged < stage_slots<NJ>(a)) {
        uint16_t *area = stage_area<NJ>(lds, a, ln.wave);
        uint16_t *slot = area + (size_t)st.staged * a.num_cols * D;
        if (keep) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const f32x4_t x = st.acc[t][2 * j] * inv, y = st.acc[t][2 * j + 1] * inv;
            *reinterpret_cast<u32x4_t *>(slot + ((j * 4 + ln.grp) * a.num_cols + ln.col[t]) * 8) =
                u32x4_t{to_bf16x2(x[0], x[1]), to_bf16x2(x[2], x[3]), to_bf16x2(y[0], y[1]), to_bf16x2(y[2], y[3])};
          }
        }
        if (ln.lane == 0) stage_dsts<NJ>(area, a)[st.staged] = dst;
        ++st.staged;
      } else if (keep) {
        store_out<NJ>(a.out + dst + ln.out_off[t], st.acc[t], inv);
      }
    } else {
      const int slot = P.first ? 0 : 1;
      if (DF && P.first) {  // kept in registers until the stream ends
        st.first_cut = keep;
#pragma unroll
        for (int k = 0; k < 2 * NJ; ++k) st.first_acc[k] = st.acc[t][k];
        st.first_m = st.m_run[t];
        st.first_l = l;
      } else if (keep) {
        // With two tiles, two scalar stores for max and sum: building a float2
        // from m_run[t] lets the compiler widen that read over m_run[t + 1],
        // which pins the array to scratch, and every reload then waits for all
        // loads in flight.
        store_record<NJ, NT>(a, ln, t, slot, st.acc[t], st.m_run[t], l);
      }
    }
  }
  if (P.first) {
    int2 d = {-1, -1};
    if (!whole && P.off + P.cnt == P.L) {  // ends a segment begun in an earlier workgroup
      const int w0 = owner_of(P.seg_start, ln.U, ln.E);
      const int slot0 = range_lo(w0, ln.U, ln.E) < P.seg_start ? 1 : 0;
      d = int2{P.s * ln.NG + P.hg, w0 * 2 + slot0};
    }
    // Sharing-aware decode also records the segment's q rows, so the merge
    // needs no read of the plan.
    if constexpr (DF) st.desc = d;
    else if (ln.tid == 0 && a.merge_desc)
      a.merge_desc[ln.w] = M == kShared ? int4{d.x, d.y, P.qrow, P.ntok} : int4{d.x, d.y, 0, 0};
  }
}

// After the stream (launches that defer): the staged whole-segment outputs,
// the first piece's partial record (if that piece was cut) and the merge
// record.
template <int NJ, int NT, int M, bool DF>
__device__ __forceinline__ void finish_stream(const DecodeArgs &a, const Lane<NT> &ln, const Stream<NJ, NT> &st,
                                              uint16_t *lds) {
  constexpr int D = NJ * 32;
  if constexpr (M == kStep) {
    // The staged new rows: lanes 0 .. D/8 - 1 store the K row, the next D/8
    // lanes the V row, 16 bytes each.
    const uint16_t *area = new_area<NJ>(lds, a, ln.wave);
    for (int i = 0; i < st.nnew; ++i) {
      const uint16_t *slot = area + (size_t)i * new_slot_elems<D>();
      const size_t dst = *reinterpret_cast<const size_t *>(slot + 2 * D);
      if (ln.lane < D / 4) {
        const int half = ln.lane / (D / 8), piece = ln.lane - half * (D / 8);
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(slot + half * D + piece * 8);
        *reinterpret_cast<u32x4_t *>(const_cast<uint16_t *>(half ? a.v_cache : a.k_cache) + dst + piece * 8) = v;
      }
    }
  }
  if constexpr (DF) {
    const uint16_t *area = stage_area<NJ>(lds, a, ln.wave);
    const size_t *dsts = stage_dsts<NJ>(const_cast<uint16_t *>(area), a);
    for (int i = 0; i < st.staged; ++i) {
      const uint16_t *slot = area + (size_t)i * a.num_cols * D;
      uint16_t *dst = a.out + dsts[i] + ln.out_off[0];
      if (ln.col_ok[0]) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          *reinterpret_cast<u32x4_t *>(dst + 32 * j) =
              *reinterpret_cast<const u32x4_t *>(slot + ((j * 4 + ln.grp) * a.num_cols + ln.col[0]) * 8);
      }
    }
    if (st.first_cut) store_record<NJ, NT>(a, ln, 0, 0, st.first_acc, st.first_m, st.first_l);
    if (ln.tid == 0 && a.merge_desc) a.merge_desc[ln.w] = int4{st.desc.x, st.desc.y, 0, 0};
  }
}

// One query head per KV head, on the vector ALU (the launch's `vector`
// path). Lane (c, grp) takes token c of the chunk: its score is the dot
// product of q with the token's key over the lane's 32 head dims (8 at
// 32j + 8*grp for each j, as loaded), summed over the token's four lanes.
// Each lane keeps its own running max (base 2), sum and unnormalised output
// over the tokens it sees (token c of every chunk), in the registers the
// matrix-core path uses for its column (m_run, l_part, acc: dims 32j +
// 8*grp + 4h + r in acc[2j + h][r]); vec_fold merges the 16 token lanes when
// the piece ends. `live`: the lane's token lies before the limit (a stale
// or NaN row past it is replaced by zeros).
template <int NJ, int NT>
__device__ __forceinline__ void vec_chunk(const DecodeArgs &a, const Lane<NT> &ln, Stream<NJ, NT> &st,
                                          const u32x4_t (&K)[NJ], const u32x4_t (&V)[NJ], bool live) {
  // The bf16 pairs come out of the 16-byte registers by shuffles of the
  // 8-element vectors: a bit cast of a single extracted 32-bit element to a
  // bf16 pair is compiled (hipcc, gfx950) into a read of element 0 for every
  // element, so that form is not used.
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, K[j]);
    const bf16x8_t qb = __builtin_bit_cast(bf16x8_t, st.qv[0][j]);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kb, kb, 0, 1), __builtin_shufflevector(qb, qb, 0, 1), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kb, kb, 2, 3), __builtin_shufflevector(qb, qb, 2, 3), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kb, kb, 4, 5), __builtin_shufflevector(qb, qb, 4, 5), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kb, kb, 6, 7), __builtin_shufflevector(qb, qb, 6, 7), s, false);
  }
  s = sum_over_groups(s);
  const float z = live ? s * a.scale_log2 : -INFINITY;
  const float m_new = fmaxf(st.m_run[0], z);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;  // a lane that has seen nothing yet
  const float alpha = fast_exp2(st.m_run[0] - m_use);
  const float p = fast_exp2(z - m_use);
  st.m_run[0] = m_new;
  st.l_part[0] = st.l_part[0] * alpha + p;
  if (alpha != 1.f) {
#pragma unroll
    for (int k = 0; k < 2 * NJ; ++k) st.acc[0][k] *= alpha;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = live ? V[j][w] : 0u;
      st.acc[0][2 * j + (w >> 1)][2 * (w & 1)] += p * bf16_lo(v);
      st.acc[0][2 * j + (w >> 1)][2 * (w & 1) + 1] += p * bf16_hi(v);
    }
}

// Lane-to-lane exchange inside rows of 16 lanes (DPP).
__device__ __forceinline__ float row_dpp(float x, int ctrl) {
  switch (ctrl) {  // the control must be a constant
    case 0: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, true));
    case 1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, true));
    case 2: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xf, 0xf, true));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xf, 0xf, true));
  }
}

// The vector path at a piece's end: merges the 16 token lanes of each row
// (log-sum-exp weights, a butterfly over lane^1, lane^2 (quad permutes), the
// half-row mirror and the row mirror, after which every lane of a row holds
// the row's result), then leaves the state as the matrix-core path does:
// running max, the sum counted once per column (grp 0), unnormalised output.
template <int NJ, int NT>
__device__ __forceinline__ void vec_fold(const Lane<NT> &ln, Stream<NJ, NT> &st) {
  float m = st.m_run[0], l = st.l_part[0];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float mo = row_dpp(m, k), lo = row_dpp(l, k);
    const float M = fmaxf(m, mo);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float w1 = fast_exp2(m - Mu), w2 = fast_exp2(mo - Mu);
    l = l * w1 + lo * w2;
#pragma unroll
    for (int i = 0; i < 2 * NJ; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) st.acc[0][i][r] = st.acc[0][i][r] * w1 + row_dpp(st.acc[0][i][r], k) * w2;
    m = M;
  }
  st.m_run[0] = m;
  st.l_part[0] = ln.grp == 0 ? l : 0.f;
}

// kStep: the newest position's K/V row of this wavefront's KV head goes to
// its slot in the cache: row (n - 1) % block_size of the physical block the
// table names for position n - 1. Lanes of tile row 0 hold it (dims 32j +
// 8*grp .. +7). It is staged in LDS and stored after the stream (a store
// issued mid-stream would make the waits for later loads wait for it too);
// past the staging capacity it is stored at once. A table entry outside the
// pool skips the write.
template <int NJ, int NT, int M, int BS>
__device__ __forceinline__ void stage_new(const int32_t *__restrict__ tables, const DecodeArgs &a, const Lane<NT> &ln,
                                          Stream<NJ, NT> &st, uint16_t *lds, const u32x4_t (&K)[NJ],
                                          const u32x4_t (&V)[NJ]) {
  constexpr int D = NJ * 32;
  const Piece &P = st.P;
  const int pos = P.n - 1;
  const int id = tables[(size_t)P.s * a.max_blocks_per_seq + pos / BS];
  if ((uint32_t)id >= ln.pool32) return;
  const size_t dst = (size_t)id * ln.blk_stride + (size_t)(pos % BS) * a.num_kv_heads * D + head_off<NJ, M>(ln, P);
  if (st.nnew < kNewSlots) {
    uint16_t *slot = new_area<NJ>(lds, a, ln.wave) + (size_t)st.nnew * new_slot_elems<D>();
    if (ln.c == 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        *reinterpret_cast<u32x4_t *>(slot + 32 * j + 8 * ln.grp) = K[j];
        *reinterpret_cast<u32x4_t *>(slot + D + 32 * j + 8 * ln.grp) = V[j];
      }
    }
    if (ln.lane == 0) *reinterpret_cast<size_t *>(slot + 2 * D) = dst;
    ++st.nnew;
  } else if (ln.c == 0) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      *reinterpret_cast<u32x4_t *>(const_cast<uint16_t *>(a.k_cache) + dst + 32 * j + 8 * ln.grp) = K[j];
      *reinterpret_cast<u32x4_t *>(const_cast<uint16_t *>(a.v_cache) + dst + 32 * j + 8 * ln.grp) = V[j];
    }
  }
}

// Makes Q the current piece (its first block is already loading) and looks
// one piece further ahead. With one column tile Q's q is in LDS already;
// with two it is loaded here, into registers or parked in LDS (q_in_regs).
template <int NJ, int NT, int M, int BS>
__device__ __forceinline__ void advance(const DecodeArgs &a, const Lane<NT> &ln, Walker &wk, Stream<NJ, NT> &st,
                                        uint16_t *lds) {
  constexpr int CH = chunk_of<BS>();
  st.P = st.Q;
  ++st.ord;
  if constexpr (NT == 1) {
    const uint16_t *qs = q_slot<NJ>(lds, a, ln.wave, st.ord) + ln.grp * 8;
#pragma unroll
    for (int j = 0; j < NJ; ++j) st.qv[0][j] = *reinterpret_cast<const u32x4_t *>(qs + ln.col[0] * q_row<NJ>() + 32 * j);
  } else if constexpr (q_in_regs<NT, M, BS>()) {
    load_q<NJ, NT, M>(a, ln, st.P, st.qv);
  } else {
    u32x4_t qv[NT][NJ];
    load_q<NJ, NT, M>(a, ln, st.P, qv);
    park_q<NJ>(q_park<NJ>(lds, a, ln.wave), ln, qv);
  }
  st.hoff = st.hoff_q;
  st.i = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    st.m_run[t] = -INFINITY;
    st.l_part[t] = 0.f;
#pragma unroll
    for (int k = 0; k < 2 * NJ; ++k) st.acc[t][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  st.has_q = next_piece<M, CH>(wk, st.Q);
  if (!st.has_q) st.Q = st.P;
  st.hoff_q = head_off<NJ, M>(ln, st.Q);
  if constexpr (M == kShared) {
    st.mv_p = st.mv_q;
    st.mv_q = member_info(wk.lens, st.Q, ln.lane, wk.cap);
  }
}

// Computes block i of P from (K, V) after starting the next block of the
// stream loading into (Kn, Vn); finishes P at its end and moves to Q.
// Returns false once the stream is done.
template <int NJ, int NT, int M, int BS, bool VEC>
__device__ __forceinline__ bool step(const int32_t *__restrict__ tables, const DecodeArgs &a, const Lane<NT> &ln,
                                     Walker &wk, Stream<NJ, NT> &st, u32x4_t (&K)[NJ], u32x4_t (&V)[NJ],
                                     u32x4_t (&Kn)[NJ], u32x4_t (&Vn)[NJ], uint16_t *lds) {
  constexpr bool kMulti = causal(M);
  constexpr int CH = chunk_of<BS>();
  const Piece &P = st.P;
  // In P's first step, q of the next piece is loaded (before this step's K/V
  // loads) and parked in LDS at the end of the step: the registers never
  // cross a loop iteration, and the wait for them covers only the K/V loads
  // issued after them.
  const bool stage_q = NT == 1 && st.i == 0 && st.has_q;
  u32x4_t qt[NT][NJ];
  if (stage_q) load_q<NJ, NT, M>(a, ln, st.Q, qt);
  // The next block of the stream: P's next, else Q's first. The loads are
  // issued on every path (past the end of the stream they reload the
  // current block, which is still in the cache), so the compiler can count
  // them when it places the wait for the current block: it waits for that
  // block only, not for the next.
  const int nx = st.i + 1;
  const bool in_p = nx < P.cnt;
  const bool to_q = !in_p && st.has_q;
  Cursor cn;
  if constexpr (M == kShared) {
    cn = in_p ? seg_next(P, st.cc, st.mv_p, ln.lane) : (to_q ? seg_first(st.Q, st.mv_q, ln.lane) : st.cc);
    issue_shared<NJ, NT, BS>(tables, a, ln, to_q ? st.Q : P, cn, to_q ? st.hoff_q : st.hoff, rows_in(cn.n, cn.b),
                             Kn, Vn);
  } else {
    const int next_s = to_q ? st.Q.s : P.s;
    const int next_b = in_p ? P.off + nx : (to_q ? st.Q.off : P.off + st.i);
    issue_seq<NJ, NT, M, BS>(tables, a, ln, next_s, next_b, to_q ? st.Q.n : P.n, to_q ? st.Q.L : P.L,
                             to_q ? st.hoff_q : st.hoff, Kn, Vn);
  }
  // Keep the scheduler from sinking those loads below the compute.
  __builtin_amdgcn_sched_barrier(0);

  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const int b = M == kShared ? st.cc.b : P.off + st.i;
  // kStep: the last chunk of a segment is the newest position alone (row 0),
  // and the cached chunks before it end at position n - 2.
  const bool fresh = M == kStep && b == P.L - 1;
  const int pos_base = fresh ? P.n - 1 : b * CH;
  const int vis = M == kStep ? (fresh ? P.n : P.n - 1) : P.n;  // positions < vis are in this chunk's rows
  const int pos0 = pos_base + ln.grp * 4;
  // kShared: the columns of the members that see the chunk (j .. e) are
  // live; a tile holding none of them is skipped (a uniform branch).
  const int cj = M == kShared ? st.cc.j : 0, ce = M == kShared ? st.cc.e : 0;
  auto tile_live = [&](int t) {
    if constexpr (M != kShared) return true;
    return cj * a.group < 16 * (t + 1) && (ce + 1) * a.group > 16 * t;
  };
  if constexpr (VEC) {
    vec_chunk<NJ>(a, ln, st, K, V, pos_base + ln.c < vis);
  } else {
  u32x2_t pb_hi[NT], pb_lo[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!tile_live(t)) continue;
    f32x4_t sc = zero4;
    if constexpr (q_in_regs<NT, M, BS>()) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) sc = mfma32(K[j], st.qv[t][j], sc);
    } else {
      u32x4_t qv[NJ];
      parked_q<NJ>(q_park<NJ>(lds, a, ln.wave), ln, t, qv);
#pragma unroll
      for (int j = 0; j < NJ; ++j) sc = mfma32(K[j], qv[j], sc);
    }
    // Positions past the column's causal limit (the context length for a
    // single new token) are masked, and so are a dead column's.
    int lim;
    if constexpr (kMulti) lim = P.n - ln.qshift[t];
    else if constexpr (M == kShared) lim = (ln.tok[t] >= cj && ln.tok[t] <= ce) ? st.cc.n : 0;
    else lim = vis;
    float z[4];
#pragma unroll
    // With 8-token chunks the tile's rows 8-15 hold no token of the chunk.
    for (int r = 0; r < 4; ++r)
      z[r] = (ln.grp * 4 + r < CH && pos0 + r < lim) ? sc[r] * a.scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mx = max_over_groups(mx);
    // With one new token, position b*16 is always visible, so the max is
    // finite. With several, a column may see nothing in this block yet.
    const float m_new = fmaxf(st.m_run[t], mx);
    const float m_use = (kMulti || M == kShared) ? (m_new == -INFINITY ? 0.f : m_new) : m_new;
    const float alpha = fast_exp2(st.m_run[t] - m_use);
    st.m_run[t] = m_new;

    // P = P_hi + P_lo, both bf16.
    const float p0 = fast_exp2(z[0] - m_use), p1 = fast_exp2(z[1] - m_use);
    const float p2 = fast_exp2(z[2] - m_use), p3 = fast_exp2(z[3] - m_use);
    const uint32_t h01 = to_bf16x2(p0, p1), h23 = to_bf16x2(p2, p3);
    pb_hi[t] = u32x2_t{h01, h23};
    pb_lo[t] = u32x2_t{to_bf16x2(p0 - bf16_lo(h01), p1 - bf16_hi(h01)), to_bf16x2(p2 - bf16_lo(h23), p3 - bf16_hi(h23))};
    st.l_part[t] = st.l_part[t] * alpha + ((p0 + p1) + (p2 + p3));
#pragma unroll
    for (int k = 0; k < 2 * NJ; ++k) st.acc[t][k] *= alpha;
  }

  // V rows of tokens at or past n must not reach the sum, even as NaN * 0.
  const bool v_live = ln.c < CH && pos_base + ln.c < (M == kShared ? st.cc.n : vis);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x2_t vin = v_live ? u32x2_t{V[j][2 * h], V[j][2 * h + 1]} : u32x2_t{0u, 0u};
      const f32x4_t tv = mfma16(vin, ln.sel, zero4);
      const u32x2_t av = {pack_hi(tv[0], tv[1]), pack_hi(tv[2], tv[3])};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (!tile_live(t)) continue;
        st.acc[t][2 * j + h] = mfma16(av, pb_hi[t], st.acc[t][2 * j + h]);
        st.acc[t][2 * j + h] = mfma16(av, pb_lo[t], st.acc[t][2 * j + h]);
      }
    }
  }
  }  // matrix-core path

  if constexpr (M == kStep) {
    if (fresh && a.write_new) stage_new<NJ, NT, M, BS>(tables, a, ln, st, lds, K, V);
  }
  if (stage_q) park_q<NJ>(q_slot<NJ>(lds, a, ln.wave, st.ord + 1), ln, qt);

  st.i = nx;
  if constexpr (M == kShared) st.cc = cn;
  if (in_p) return true;
  if constexpr (VEC) vec_fold<NJ>(ln, st);
  finish_piece<NJ, NT, M, defers<NT, BS>()>(a, ln, st, lds);
  if (!st.has_q) return false;
  advance<NJ, NT, M, BS>(a, ln, wk, st, lds);
  return true;
}

// An empty sequence attends to nothing: its output rows are zero. Done by one
// workgroup per sequence.
template <int D>
__device__ __forceinline__ void zero_empty(const DecodeArgs &a, int s, int w) {
  if (s % a.num_wgs != w) return;
  const int rows = a.q_len * a.num_q_heads;
  u32x4_t *row = reinterpret_cast<u32x4_t *>(a.out + (size_t)s * rows * D);
  for (int i = 0; i < rows * D / 8; ++i) row[i] = u32x4_t{0, 0, 0, 0};
}

// Workgroups past the ones that get units have no merge record to write.
__device__ __forceinline__ void no_merge(const DecodeArgs &a, int w, int tid) {
  if (tid == 0 && a.merge_desc) a.merge_desc[w] = int4{-1, -1, 0, 0};
}

// kShared: a segment with no chunk (every member's context empty) is not
// decoded; its members' output rows are zeroed here, segment v by workgroup
// v mod num_wgs, all threads of the workgroup together. The plan counts such
// segments, so calls without them skip this.
template <int D>
__device__ __forceinline__ void zero_empty_items(const DecodeArgs &a, const ShareItem *__restrict__ items, int nitems,
                                                 int w, int tid, int nthr) {
  const int row_vec = a.num_q_heads * D / 8;  // 16-byte vectors per q row
  for (int v = w; v < nitems; v += a.num_wgs) {
    const ShareItem x = items[v];
    if (x.L != 0 || x.qrow < 0 || x.ntok < 1 || x.ntok > a.num_seqs - x.qrow) continue;
    u32x4_t *row = reinterpret_cast<u32x4_t *>(a.out) + (size_t)x.qrow * row_vec;
    for (int k = tid; k < x.ntok * row_vec; k += nthr) row[k] = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// NT: 16-column MFMA tiles per wavefront (columns = q_len * group, or the
// item width in kShared, or 32 per column group in kWide). M: kSingle,
// kCausal, kWide or kShared. The narrow launches put one wavefront on each
// SIMD. kWide runs two wavefronts per SIMD (a workgroup of up to 8 column
// groups of one KV head), 256 registers each. Four tiles of several new
// tokens (33-64 columns), and two with 8-token blocks (two loads in flight
// per row), do not fit in 256 arch registers: those launches bound their
// workgroup at 256 threads, so a wavefront may also use accumulation
// registers (no scratch; two tiles with 8-token blocks: 282 against 286 us
// at 8 new tokens).
template <int D, int NT, int M, int BS, bool VEC>
__global__ __launch_bounds__(M == kCausal && (NT == 4 || (NT == 2 && BS == 8)) ? 256 : 512)
__attribute__((amdgpu_waves_per_eu(NT == 1 || M == kWide ? 2 : 1)))
void decode_kernel(const DecodeArgs a, const int32_t *__restrict__ tables, const int32_t *__restrict__ lens,
                   const ShareItem *__restrict__ items) {
  constexpr int NJ = D / 32;  // MFMA steps over head_size; 16-byte loads per lane per row
  static_assert(NJ >= 1 && D % 32 == 0, "head_size must be a multiple of 32");
  extern __shared__ __align__(16) uint16_t q_lds[];  // heads_per_wg * (NT == 1 ? 2 : 1) * rec_cols * (D + 8), ...
  __shared__ long long red[8];
  __shared__ int found_seq, found_n;
  __shared__ long long found_prefix;

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int lane = tid & 63;
  const int w = blockIdx.x;
  const int S = a.num_seqs;
  const int NG = a.num_head_groups;
  const int cap = a.max_blocks_per_seq * BS;  // tokens a table row can address
  constexpr int CH = chunk_of<BS>();          // tokens per chunk (unit of work)
  const long long W = a.num_wgs;

  long long U, lo, hi, E;
  Walker wk;
  int sh_items = 0, sh_empty = 0;  // kShared: the plan's segments, and those with no chunk
  if constexpr (M == kShared) {
    // The plan kernel wrote the items and their first units; one parallel
    // search finds the item that holds `lo` (empty items never match).
    ShareHeader h = *a.share;
    h.items = min(max(h.items, 0), S);  // the plan writes at most one segment per sequence
    sh_items = h.items;
    sh_empty = h.empty;
    U = h.units;
    E = U < W ? U : W;
    if (w >= E) {  // every workgroup writes its merge record, this one "none"
      if (sh_empty > 0) zero_empty_items<D>(a, items, sh_items, w, tid, nthr);
      no_merge(a, w, tid);
      return;
    }
    lo = range_lo(w, U, E);
    hi = range_lo(w + 1, U, E);
    if (tid == 0) found_seq = -1;
    __syncthreads();
    for (int v = tid; v < h.items; v += nthr)
      if (items[v].ustart <= lo && lo < items[v + 1].ustart) found_seq = v;
    __syncthreads();
    if (found_seq < 0) {  // only if the plan is inconsistent
      no_merge(a, w, tid);
      return;
    }
    const int v = __builtin_amdgcn_readfirstlane(found_seq);
    wk.items = items;
    wk.lens = lens;
    wk.cap = cap;
    wk.S = h.items;
    wk.S_rows = S;
    take_item(wk, items[v]);
    wk.s = v;
    const long long us = items[v].ustart;
    wk.seg_base = (long long)(((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane((int)(us >> 32)) << 32) |
                              (unsigned)__builtin_amdgcn_readfirstlane((int)us));
  } else if (S <= nthr) {
    // One pass: every thread holds one sequence's block count; a block scan
    // gives the total and every sequence's first unit at once.
    const int n = tid < S ? clamp_len(lens[tid], cap) : 0;
    if (tid < S && n == 0) zero_empty<D>(a, tid, w);
    const long long L = seg_chunks<M, CH>(n);
    long long pre, total;
    const long long incl = wg_scan(L, red, wave, lane, nthr >> 6, pre, total);
    U = total * NG;
    E = U < W ? U : W;  // workgroups that get units
    if (w >= E) {
      no_merge(a, w, tid);
      return;
    }
    lo = range_lo(w, U, E);
    hi = range_lo(w + 1, U, E);
    const long long excl = pre + incl - L;
    if (L > 0 && excl * NG <= lo && lo < (excl + L) * NG) {
      found_seq = tid;
      found_prefix = excl;
      found_n = n;
    }
    __syncthreads();
  } else {
    // More sequences than threads: each thread takes a contiguous range of K
    // of them. It sums their units with a tile of loads in flight at once
    // (a loop of dependent rounds, one per sequence block, measured 60-90 us
    // at 4096 sequences with one wavefront per workgroup); one scan over the
    // threads then gives the call's total and every range's first unit, and
    // the thread whose range holds `lo` reads its range again, from cache, to
    // find the sequence. The loads go through a buffer resource over the S
    // lengths, so the tail past S reads zeros.
    constexpr int kTile = 16;
    const int K = (S + nthr - 1) / nthr;
    const int s0 = min(tid * K, S), s1 = min(s0 + K, S);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t *>(lens), 0, (int)((uint32_t)S * sizeof(int32_t)), kRawBufferWord3);
    long long mine = 0;
    for (int s = s0; s < s1; s += kTile) {
      int nv[kTile];
#pragma unroll
      for (int k = 0; k < kTile; ++k) nv[k] = (int)__builtin_amdgcn_raw_buffer_load_b32(rl, (s + k) * 4, 0, 0);
#pragma unroll
      for (int k = 0; k < kTile; ++k) {
        if (s + k < s1) {
          const int n = clamp_len(nv[k], cap);
          mine += seg_chunks<M, CH>(n);
          if (n == 0) zero_empty<D>(a, s + k, w);
        }
      }
    }
    long long pre, total;
    const long long incl = wg_scan(mine, red, wave, lane, nthr >> 6, pre, total);
    U = total * NG;
    E = U < W ? U : W;
    if (w >= E) {
      no_merge(a, w, tid);
      return;
    }
    lo = range_lo(w, U, E);
    hi = range_lo(w + 1, U, E);
    if (tid == 0) found_seq = -1;
    __syncthreads();
    long long acc = pre + incl - mine;  // the first chunk of this thread's range
    if (mine > 0 && acc * NG <= lo && lo < (acc + mine) * NG) {
      bool done = false;
      for (int s = s0; s < s1 && !done; s += kTile) {
        int nv[kTile];
#pragma unroll
        for (int k = 0; k < kTile; ++k) nv[k] = (int)__builtin_amdgcn_raw_buffer_load_b32(rl, (s + k) * 4, 0, 0);
#pragma unroll
        for (int k = 0; k < kTile; ++k) {
          if (done || s + k >= s1) continue;
          const int n = clamp_len(nv[k], cap);
          const long long L = seg_chunks<M, CH>(n);
          if (L > 0 && acc * NG <= lo && lo < (acc + L) * NG) {
            found_seq = s + k;
            found_prefix = acc;
            found_n = n;
            done = true;
          }
          acc += L;
        }
      }
    }
    __syncthreads();
    if (found_seq < 0) {  // only if the lengths changed during the call
      no_merge(a, w, tid);
      return;
    }
  }

  if constexpr (M != kShared) {
    wk.lens = lens;
    wk.S = S;
    wk.cap = cap;
    wk.seg_base = found_prefix * NG;
    wk.s = __builtin_amdgcn_readfirstlane(found_seq);
    wk.n = __builtin_amdgcn_readfirstlane(found_n);
    wk.L = seg_chunks<M, CH>(wk.n);
  }
  wk.NG = NG;
  wk.u = lo;
  wk.hi = hi;
  wk.hg = (int)((lo - wk.seg_base) / wk.L);
  wk.off = (int)((lo - wk.seg_base) % wk.L);
  wk.first = true;

  // The wavefront serves KV head hg*HG + wave of every piece. Its columns are
  // (new token, query head of that KV head's group) pairs; lanes whose column
  // does not exist repeat the last column, and their results are never
  // stored.
  Lane<NT> ln;
  ln.tid = tid;
  ln.wave = wave;
  ln.lane = lane;
  ln.c = lane & 15;
  ln.grp = lane >> 4;
  ln.w = w;
  ln.HG = a.heads_per_wg;
  ln.NG = NG;
  // kWide: wavefront w holds columns 32*w .. 32*w + 31 of its KV head.
  const int col0 = M == kWide ? 32 * wave : 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = col0 + 16 * t + ln.c;
    ln.col_ok[t] = col < a.num_cols;
    ln.col[t] = ln.col_ok[t] ? col : a.num_cols - 1;
    ln.lcol[t] = ln.col[t] - col0;
    const int tok = ln.col[t] / a.group;
    const int qh = ln.col[t] - tok * a.group;
    ln.qshift[t] = a.q_len - 1 - tok;
    ln.tok[t] = tok;
    ln.out_off[t] = (uint32_t)((tok * a.num_q_heads + qh) * D + ln.grp * 8);
    ln.q_off[t] = ln.out_off[t] * (uint32_t)sizeof(uint16_t);
  }
  ln.blk_stride = (size_t)a.num_kv_heads * D * BS;
  ln.row_bytes = a.num_kv_heads * D * (int)sizeof(uint16_t);
  ln.lane_off = (uint32_t)(((size_t)ln.c * a.num_kv_heads * D + ln.grp * 8) * sizeof(uint16_t));
  ln.lane_off_b = ln.c >= kBlock / 2 ? ln.lane_off - (uint32_t)(kBlock / 2 * ln.row_bytes) : 0x80000000u;
  ln.U = U;
  ln.E = E;
  ln.pool32 = (uint32_t)(a.num_blocks < 0x7fffffffLL ? a.num_blocks : 0x7fffffffLL);
  // One-hot selector: lane (c, grp) holds 1.0 in element c%4 iff grp == c/4.
  ln.sel = u32x2_t{0u, 0u};
  if (ln.grp == (ln.c >> 2)) {
    const uint32_t word = (ln.c & 1) ? (kBf16One << 16) : kBf16One;
    if (ln.c & 2) ln.sel.y = word; else ln.sel.x = word;
  }

  // Software pipeline over the workgroup's stream of blocks. Two register
  // buffers take turns: while one block is computed, the next block of the
  // stream (possibly the first block of the next piece) loads into the
  // other. The next piece's q goes through LDS one piece ahead.
  Stream<NJ, NT> st;
  next_piece<M, CH>(wk, st.P);
  if constexpr (q_in_regs<NT, M, BS>()) {
    load_q<NJ, NT, M>(a, ln, st.P, st.qv);
  } else {
    u32x4_t qv[NT][NJ];
    load_q<NJ, NT, M>(a, ln, st.P, qv);
    park_q<NJ>(q_park<NJ>(q_lds, a, wave), ln, qv);
  }
  st.hoff = head_off<NJ, M>(ln, st.P);
  st.has_q = next_piece<M, CH>(wk, st.Q);
  if (!st.has_q) st.Q = st.P;
  st.hoff_q = head_off<NJ, M>(ln, st.Q);
  if constexpr (M == kShared) {
    st.mv_p = member_info(lens, st.P, lane, cap);
    st.mv_q = member_info(lens, st.Q, lane, cap);
    st.cc = seg_first(st.P, st.mv_p, lane);
  }
  st.i = 0;
  st.ord = 0;
  st.first_cut = false;
  st.desc = int2{-1, -1};
  st.staged = 0;
  st.nnew = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    st.m_run[t] = -INFINITY;
    st.l_part[t] = 0.f;
#pragma unroll
    for (int k = 0; k < 2 * NJ; ++k) st.acc[t][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  u32x4_t KA[NJ], VA[NJ], KB[NJ], VB[NJ];
  if constexpr (M == kShared) {
    issue_shared<NJ, NT, BS>(tables, a, ln, st.P, st.cc, st.hoff, rows_in(st.cc.n, st.cc.b), KA, VA);
  } else {
    issue_seq<NJ, NT, M, BS>(tables, a, ln, st.P.s, st.P.off, st.P.n, st.P.L, st.hoff, KA, VA);
  }
  while (step<NJ, NT, M, BS, VEC>(tables, a, ln, wk, st, KA, VA, KB, VB, q_lds) &&
         step<NJ, NT, M, BS, VEC>(tables, a, ln, wk, st, KB, VB, KA, VA, q_lds)) {
  }
  finish_stream<NJ, NT, M, defers<NT, BS>()>(a, ln, st, q_lds);
  if constexpr (M == kShared) {
    if (sh_empty > 0) zero_empty_items<D>(a, items, sh_items, w, tid, nthr);
  }
}

// Log-sum-exp merge of the pieces of segments cut by workgroup boundaries.
// Grid: one block per decode workgroup w, one wavefront per wavefront of the
// decode workgroup (a KV head of a head group, or a column group). Block w merges the segment that workgroup w's first piece
// ended, if any (the others exit at once). Lanes take 8 head dims of a column
// each (D/8 lanes per column) and two columns per pass, 64 / (D/8) columns
// apart. The pieces are slot d.y & 1 of workgroup d.y >> 1, then the first
// slot of every workgroup up to w; the records of four pieces of both columns
// are loaded together, then folded in with a running rescale.
template <int D, bool kSegments>
__global__ __launch_bounds__(512) void merge_kernel(const DecodeArgs a) {
  constexpr int LPC = D / 8;     // lanes per column
  constexpr int CPP = 64 / LPC;  // columns per half pass
  constexpr int kPieces = 4;
  const int w1 = blockIdx.x;
  const int4 d = a.merge_desc[w1];
  if (d.x < 0) return;
  // Every index below comes from the workspace. Each is checked before it
  // is used, so a bookkeeping slip gives a wrong result, never an access
  // outside the call's arrays: the segment must be one of the call's (in
  // sharing-aware decode its q rows must lie in the batch), and its first
  // piece must belong to this workgroup or an earlier one.
  if (d.x >= a.num_seqs * a.num_head_groups || d.y < 0 || (d.y >> 1) > w1) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // KV head within the head group
  const int lane = threadIdx.x & 63;
  const int HG = a.heads_per_wg;
  const int s = d.x / a.num_head_groups;
  // The wavefront's KV head and column group: one head per wavefront, or
  // (more than 32 columns) the head group's one head with the wavefront's
  // 32 columns.
  const int vh = (d.x - s * a.num_head_groups) * HG + wave;
  const int g = vh / a.col_groups;
  const int col0 = (vh - g * a.col_groups) * a.rec_cols;
  // Output rows: the sequence's q_len rows, or a segment's members (kSegments).
  size_t row0 = (size_t)s * a.q_len;
  int cols = min(a.rec_cols, a.num_cols - col0);
  if constexpr (kSegments) {
    const int qrow = d.z, ntok = d.w;
    if (qrow < 0 || ntok < 1 || ntok > a.num_seqs - qrow || ntok * a.group > a.num_cols) return;
    row0 = (size_t)qrow;
    cols = ntok * a.group;
  }
  const float *__restrict__ pml = a.part_ml;
  const float *__restrict__ pob = a.part_o;
  const int w0 = d.y >> 1;
  const int sub = lane / LPC, dd = (lane - sub * LPC) * 8;
  for (int c0 = 0; c0 < cols; c0 += 2 * CPP) {
    float Mx[2] = {-INFINITY, -INFINITY}, Ls[2] = {0.f, 0.f};
    f32x4_t o[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) o[u][0] = o[u][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int w = w0; w <= w1; w += kPieces) {
      float pm[2][kPieces], pl[2][kPieces];
      f32x4_t po[2][kPieces][2];
#pragma unroll
      for (int k = 0; k < kPieces; ++k) {
        const size_t rec = w + k == w0 ? (size_t)d.y : (size_t)2 * (w + k);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = c0 + u * CPP + sub;
          pm[u][k] = -INFINITY;  // padding: weight 0
          pl[u][k] = 0.f;
          po[u][k][0] = po[u][k][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (w + k <= w1 && c < cols) {
            const size_t r = (rec * HG + wave) * a.rec_cols + c;
            const f32x2_t ml = *reinterpret_cast<const f32x2_t *>(pml + r * 2);
            pm[u][k] = ml[0];
            pl[u][k] = ml[1];
            po[u][k][0] = *reinterpret_cast<const f32x4_t *>(pob + r * D + dd);
            po[u][k][1] = *reinterpret_cast<const f32x4_t *>(pob + r * D + dd + 4);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float Mn = Mx[u];
#pragma unroll
        for (int k = 0; k < kPieces; ++k) Mn = fmaxf(Mn, pm[u][k]);
        // A piece may see no position of a column (several new tokens, an
        // empty member): its max is -inf and its weight 0; so is the running
        // max before the first piece.
        const float Mu = Mn == -INFINITY ? 0.f : Mn;
        const float so = fast_exp2(Mx[u] - Mu);
        Ls[u] *= so;
        o[u][0] = o[u][0] * so;
        o[u][1] = o[u][1] * so;
#pragma unroll
        for (int k = 0; k < kPieces; ++k) {
          const float wt = fast_exp2(pm[u][k] - Mu);
          Ls[u] += wt * pl[u][k];
          o[u][0] += po[u][k][0] * wt;
          o[u][1] += po[u][k][1] * wt;
        }
        Mx[u] = Mn;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * CPP + sub;
      if (c >= cols) continue;
      const float inv = Ls[u] > 0.f ? 1.f / Ls[u] : 0.f;
      const int tok = (col0 + c) / a.group, qh = col0 + c - tok * a.group;
      const f32x4_t x = o[u][0] * inv, y = o[u][1] * inv;
      const u32x4_t v = {to_bf16x2(x[0], x[1]), to_bf16x2(x[2], x[3]), to_bf16x2(y[0], y[1]), to_bf16x2(y[2], y[3])};
      *reinterpret_cast<u32x4_t *>(a.out + ((row0 + tok) * a.num_q_heads + (size_t)g * a.group + qh) * D + dd) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Sharing-aware decode: sequences in a group share the leading blocks of
// their tables (parallel samples share the prompt, beams their history:
// "vLLM: Anatomy and Mechanisms", section "Memory Sharing via Copy-on-Write
// (CoW)"; prompts with a common beginning reuse cached blocks: section
// "Prefix Caching"). Those blocks are read once for up to 32 / group members
// (their query heads become MFMA columns of one segment), then each member's
// own blocks for it alone, in one stream: the softmax state runs across the
// whole segment, so no extra pass combines the shared and the own parts.
// ---------------------------------------------------------------------------

// Inclusive max-scan over the workgroup (plan kernel only).
__device__ __forceinline__ int wg_max_scan(int v, int *red, int wave, int lane, int nwaves, int &total) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v = max(v, u);
  }
  __syncthreads();
  if (lane == 63) red[wave] = v;
  __syncthreads();
  int pre = -1;
  total = -1;
  for (int i = 0; i < nwaves; ++i) {
    if (i < wave) pre = max(pre, red[i]);
    total = max(total, red[i]);
  }
  return max(v, pre);
}

// Builds the call's segments in one workgroup.
// Group form (shared_prev null):
//   * group_starts must not decrease and must stay within 0..S; otherwise no
//     group is formed and every sequence reads its own table.
//   * A sequence's group is the last one that starts at or before it (a
//     max-scan of start marks), if the sequence lies before its end.
//   * A group's shared blocks eb are clamped to 0..max_blocks_per_seq and to
//     the whole blocks each member fills; e = eb * block_size / 16 chunks.
//   * Each run of members_per_item consecutive members of a group, and each
//     sequence in no group, is one segment. Its first member reads all its
//     chunks (those before e through the group's first member's table), the
//     others their chunks from e on.
// Chain form (shared_prev given):
//   * Sequence i > 0 holds c_i chunks in common with sequence i - 1: the
//     declared blocks clamped to 0..max_blocks_per_seq and to the whole
//     blocks both fill, times block_size / 16, rounded down.
//   * A run is a maximal range of sequences each holding c_i > 0 chunks in
//     common with the one before (its start a max-scan of the breaks); each
//     members_per_item consecutive members of a run are one segment. Its
//     first member reads all its chunks, member i the others from c_i on.
// Both forms: units follow segment order, head group major within a segment.
// A segment with no chunk at all (every member's context empty) is not
// decoded: the header counts them, and the decode kernel zeroes their
// members' rows. Each sequence's record (context length, chunks before its
// own) goes to `members` for the decode. Nothing here depends on q, the
// caches or the output, so one plan serves every layer of a step.
template <int kThreads>
__global__ __launch_bounds__(kThreads) void share_plan_kernel(const SharePlanArgs p) {
  // grp[S], sid[S], own[S], len[S], shb[G], gs[G + 1], then csum[S] (64-bit)
  extern __shared__ __align__(16) int plan_lds[];
  __shared__ long long red[kThreads / 64];
  __shared__ int redi[kThreads / 64];
  __shared__ int bad, empties;
  constexpr int nwaves = kThreads / 64;
  const bool chain = p.shared_prev != nullptr;
  const int S = p.num_seqs, NGr = chain ? 0 : p.num_groups, C = p.members_per_item;
  int *grp = plan_lds;
  int *sid = grp + S;
  int *own = sid + S;
  int *len = own + S;
  int *shb = len + S;
  int *gs = shb + NGr;
  long long *csum = reinterpret_cast<long long *>(plan_lds + ((4 * S + 2 * NGr + 1 + 1) & ~1));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bs = p.block_size;
  const int cap = p.max_blocks_per_seq * bs;

  // Every input into LDS first: their loads are independent, so the plan
  // waits for memory once.
  if (tid == 0) bad = empties = 0;
  for (int i = tid; i < S; i += kThreads) {
    grp[i] = -1;
    len[i] = clamp_len(p.lens[i], cap);
    if (chain) own[i] = p.shared_prev[i];
  }
  if (NGr > 0)  // with no groups the arrays may be null
    for (int g = tid; g <= NGr; g += kThreads) gs[g] = p.group_starts[g];
  for (int g = tid; g < NGr; g += kThreads) shb[g] = min(max(p.shared_blocks[g], 0), p.max_blocks_per_seq);
  __syncthreads();

  // Per sequence: the chunks it reads through a predecessor (own) and
  // whether it opens a segment (sid, 0 or 1, until the scan below).
  if (chain) {
    // Chunks held in common with the sequence before; a sequence holding
    // none starts a run (grp: the run's start after the max-scan).
    for (int i = tid; i < S; i += kThreads) {
      const int blocks = i > 0 ? min(min(max(own[i], 0), p.max_blocks_per_seq), min(len[i], len[i - 1]) / bs) : 0;
      const int c = blocks * bs / kBlock;
      own[i] = c;
      grp[i] = c > 0 ? -1 : i;
    }
  } else {
    for (int g = tid; g < NGr; g += kThreads) {
      const int lo = gs[g], hi = gs[g + 1];
      if (lo > hi || (g == 0 && lo < 0) || (g == NGr - 1 && hi > S)) bad = 1;
    }
    __syncthreads();
    const bool valid = bad == 0;
    for (int g = tid; g < NGr; g += kThreads) {
      const int lo = gs[g], hi = gs[g + 1];
      if (valid && hi > lo) grp[lo] = g;  // distinct starts: groups are nonempty and ordered
    }
  }
  __syncthreads();
  int carry = -1;
  for (int base = 0; base < S; base += kThreads) {
    const int i = base + tid;
    int total;
    const int v = max(wg_max_scan(i < S ? grp[i] : -1, redi, wave, lane, nwaves, total), carry);
    if (i < S) grp[i] = v;
    carry = max(carry, total);
  }
  __syncthreads();
  if (chain) {
    for (int i = tid; i < S; i += kThreads) {
      const bool opens = (i - grp[i]) % C == 0;
      sid[i] = opens ? 1 : 0;
      if (opens) own[i] = 0;
    }
  } else {
    for (int i = tid; i < S; i += kThreads) {
      const int g = grp[i];
      if (g < 0) continue;
      if (i >= gs[g + 1]) {
        grp[i] = -1;
        continue;
      }
      atomicMin(&shb[g], len[i] / bs);  // LDS atomic: shared cache blocks
    }
    __syncthreads();
    for (int i = tid; i < S; i += kThreads) {
      const int g = grp[i];
      const bool opens = g < 0 || (i - gs[g]) % C == 0;
      sid[i] = opens ? 1 : 0;
      own[i] = opens ? 0 : shb[g] * bs / kBlock;
    }
  }
  __syncthreads();

  // Segment index of every sequence and the chunks of the stream up to it;
  // each sequence's record for the decode.
  long long segs_before = 0, blocks_before = 0;
  for (int base = 0; base < S; base += kThreads) {
    const int i = base + tid;
    long long opens = 0, adds = 0;
    if (i < S) {
      opens = sid[i];
      adds = (len[i] + kBlock - 1) / kBlock - own[i];
      p.members[2 * i] = len[i];
      p.members[2 * i + 1] = own[i];
    }
    long long pre, tot, preb, totb;
    const long long incl = wg_scan(opens, red, wave, lane, nwaves, pre, tot);
    const long long inclb = wg_scan(adds, red, wave, lane, nwaves, preb, totb);
    if (i < S) {
      sid[i] = (int)(segs_before + pre + incl - 1);
      csum[i] = blocks_before + preb + inclb;
    }
    segs_before += tot;
    blocks_before += totb;
  }
  __syncthreads();
  const long long NG = p.num_head_groups;
  for (int i = tid; i < S; i += kThreads) {
    if (i > 0 && sid[i] == sid[i - 1]) continue;  // not the first member of its segment
    int ntok = 1;
    while (ntok < C && i + ntok < S && sid[i + ntok] == sid[i]) ++ntok;
    const long long start = i > 0 ? csum[i - 1] : 0;
    const long long blocks = csum[i + ntok - 1] - start;
    const int g = chain ? -1 : grp[i];
    const int eb = g >= 0 ? shb[g] : 0;
    const int e = eb * bs / kBlock;
    ShareItem x;
    x.row = g >= 0 ? gs[g] : i;
    x.qrow = i;
    x.ntok = ntok;
    x.b0 = e;
    x.n = e * kBlock;
    x.eb = eb;
    x.L = (int)blocks;
    x.ustart = NG * start;
    p.items[sid[i]] = x;
    if (blocks == 0) atomicAdd(&empties, 1);  // LDS atomic: a segment with no chunk
  }
  __syncthreads();
  if (tid == 0) {
    const long long units = NG * blocks_before;
    ShareItem x = {0, 0, 0, 0, 0, 0, units, 0};
    p.items[segs_before] = x;  // sentinel: the end of the last segment
    ShareHeader h;
    h.units = units;
    h.items = (int)segs_before;
    h.empty = empties;
    *p.share = h;
  }
}

// Lets a kernel use more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per
// compute unit).
// Raises a kernel's dynamic LDS limit when a launch needs more than 48 KiB.
// The largest limit set so far is remembered per (device, kernel), so a
// repeated launch makes no runtime call besides the launch itself (which
// keeps it capturable in a graph once an eager call has run).
template <typename Kernel>
hipError_t allow_lds(Kernel kernel, size_t bytes) {
  if (bytes <= 48 * 1024) return hipSuccess;
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, size_t> allowed;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_pair(dev, reinterpret_cast<const void *>(kernel));
  std::lock_guard<std::mutex> lock(mu);
  auto it = allowed.find(key);
  if (it != allowed.end() && it->second >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(key.second, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) allowed[key] = bytes;
  return e;
}

template <int D, int NT, int M, int BS = 16, bool VEC = false>
hipError_t launch_decode_kernel(const DecodeArgs &args, size_t lds, hipStream_t stream) {
  hipError_t e = allow_lds(decode_kernel<D, NT, M, BS, VEC>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<D, NT, M, BS, VEC>), dim3((unsigned)args.num_wgs),
                     dim3(64 * (unsigned)args.heads_per_wg), lds, stream, args, args.block_tables,
                     args.context_lens, args.items);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs &args, size_t lds, hipStream_t stream) {
  // One query head per KV head: the vector path when the host chose it.
  const bool vec = args.vector_path && args.num_cols == 1;
  if (args.k_new) {
    if (vec) {
      if (args.block_size == 8) return launch_decode_kernel<D, 1, kStep, 8, true>(args, lds, stream);
      if (args.block_size == 32) return launch_decode_kernel<D, 1, kStep, 32, true>(args, lds, stream);
      return launch_decode_kernel<D, 1, kStep, 16, true>(args, lds, stream);
    }
    if (args.block_size == 8) return launch_decode_kernel<D, 1, kStep, 8>(args, lds, stream);
    if (args.block_size == 32) return launch_decode_kernel<D, 1, kStep, 32>(args, lds, stream);
    return launch_decode_kernel<D, 1, kStep>(args, lds, stream);
  }
  if (args.q_len == 1) {
    if (vec) {
      if (args.block_size == 8) return launch_decode_kernel<D, 1, kSingle, 8, true>(args, lds, stream);
      if (args.block_size == 32) return launch_decode_kernel<D, 1, kSingle, 32, true>(args, lds, stream);
      return launch_decode_kernel<D, 1, kSingle, 16, true>(args, lds, stream);
    }
    if (args.block_size == 8) return launch_decode_kernel<D, 1, kSingle, 8>(args, lds, stream);
    if (args.block_size == 32) return launch_decode_kernel<D, 1, kSingle, 32>(args, lds, stream);
    return launch_decode_kernel<D, 1, kSingle>(args, lds, stream);
  }
  if (args.num_cols <= 16) {
    if (args.block_size == 8) return launch_decode_kernel<D, 1, kCausal, 8>(args, lds, stream);
    if (args.block_size == 32) return launch_decode_kernel<D, 1, kCausal, 32>(args, lds, stream);
    return launch_decode_kernel<D, 1, kCausal>(args, lds, stream);
  }
  if (args.num_cols <= 32) {
    if (args.block_size == 8) return launch_decode_kernel<D, 2, kCausal, 8>(args, lds, stream);
    if (args.block_size == 32) return launch_decode_kernel<D, 2, kCausal, 32>(args, lds, stream);
    return launch_decode_kernel<D, 2, kCausal>(args, lds, stream);
  }
  if (args.num_cols <= kMaxNarrowCols) {
    if (args.block_size == 8) return launch_decode_kernel<D, 4, kCausal, 8>(args, lds, stream);
    if (args.block_size == 32) return launch_decode_kernel<D, 4, kCausal, 32>(args, lds, stream);
    return launch_decode_kernel<D, 4, kCausal>(args, lds, stream);
  }
  if (args.block_size == 8) return launch_decode_kernel<D, 2, kWide, 8>(args, lds, stream);
  if (args.block_size == 32) return launch_decode_kernel<D, 2, kWide, 32>(args, lds, stream);
  return launch_decode_kernel<D, 2, kWide>(args, lds, stream);
}

}  // namespace

int32_t decode_stage_slots(int32_t num_cols, int32_t head_size, int32_t block_size, bool new_rows) {
  if (num_cols > 16 || block_size == 8) return 0;
  const int q_ring = 2 * num_cols * (head_size + 8) * (int)sizeof(uint16_t);
  const int avail = kLdsPerWave - q_ring - (new_rows ? kNewSlots * (4 * head_size + 16) : 0);
  int n = avail > 0 ? avail / (stage_out_bytes(1, num_cols, head_size) + 8) : 0;
  if (n > kMaxStageSlots) n = kMaxStageSlots;
  while (n > 0 && stage_stride(n, num_cols, head_size) > avail) --n;
  return n;
}

hipError_t launch_decode(const DecodeArgs &args, int32_t head_size, hipStream_t stream) {
  const bool wide = args.num_cols > kMaxNarrowCols;
  const bool fused = args.k_new != nullptr;
  if (args.q_len < 1 || args.num_cols > kMaxDecodeCols || (args.q_len == 1 && args.num_cols > 16)) return hipErrorInvalidValue;
  if (fused && (args.q_len != 1 || !args.v_new)) return hipErrorInvalidValue;
  // Columns per wavefront: all of them, or (wide) 32 per column group with
  // one wavefront per column group of the head group's one KV head.
  if (wide ? (args.rec_cols != 32 || args.col_groups != (args.num_cols + 31) / 32 ||
              args.heads_per_wg != args.col_groups || args.num_head_groups != args.num_kv_heads)
           : (args.rec_cols != args.num_cols || args.col_groups != 1))
    return hipErrorInvalidValue;
  if (args.block_size != 8 && args.block_size != 16 && args.block_size != 32) return hipErrorInvalidValue;
  if (head_size != 128 && head_size != 64) return hipErrorInvalidValue;
  // LDS per wavefront: q, as a two-slot ring for the next piece (one column
  // tile) or the current piece's (two tiles); with the fused step the new
  // K/V rows staged for their slots; with one column tile (not 8-token
  // blocks) an output staging area in the room left of kLdsPerWave.
  const int q_ring = (args.num_cols <= 16 ? 2 : 1) * args.rec_cols * (head_size + 8) * (int)sizeof(uint16_t);
  const bool writes = fused && args.write_new;
  const int new_rows = writes ? kNewSlots * (4 * head_size + 16) : 0;
  DecodeArgs a = args;
  a.stage_slots = decode_stage_slots(args.num_cols, head_size, args.block_size, writes);
  const size_t lds =
      (size_t)args.heads_per_wg * (q_ring + stage_stride(a.stage_slots, args.num_cols, head_size) + new_rows);
  hipError_t err = head_size == 128 ? launch_decode_d<128>(a, lds, stream) : launch_decode_d<64>(a, lds, stream);
  if (err != hipSuccess || args.num_wgs <= 1) return err;
  const dim3 mgrid((unsigned)args.num_wgs);
  const dim3 mblock(64 * (unsigned)args.heads_per_wg);
  if (head_size == 128) {
    hipLaunchKernelGGL((merge_kernel<128, false>), mgrid, mblock, 0, stream, args);
  } else {
    hipLaunchKernelGGL((merge_kernel<64, false>), mgrid, mblock, 0, stream, args);
  }
  return hipGetLastError();
}

hipError_t launch_share_plan(const SharePlanArgs &plan, hipStream_t stream) {
  if (!plan.members || !plan.lens || !plan.items || !plan.share ||
      (plan.block_size != 8 && plan.block_size != 16 && plan.block_size != 32) || plan.num_seqs < 1 ||
      plan.num_seqs > kMaxSharedSeqs || plan.num_groups < 0 || plan.num_groups > plan.num_seqs ||
      plan.members_per_item < 1 || plan.num_head_groups < 1)
    return hipErrorInvalidValue;
  constexpr int kPlanThreads = 512;
  const size_t plan_lds =
      ((4 * (size_t)plan.num_seqs + 2 * (size_t)(plan.shared_prev ? 0 : plan.num_groups) + 2) & ~(size_t)1) *
          sizeof(int) +
      (size_t)plan.num_seqs * sizeof(long long);
  hipError_t e = allow_lds(share_plan_kernel<kPlanThreads>, plan_lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(share_plan_kernel<kPlanThreads>, dim3(1), dim3(kPlanThreads), plan_lds, stream, plan);
  return hipGetLastError();
}

hipError_t launch_decode_planned(const DecodeArgs &args, int32_t head_size, hipStream_t stream) {
  if (args.q_len != 1 || (args.block_size != 8 && args.block_size != 16 && args.block_size != 32) ||
      args.num_cols <= 16 || args.num_cols > 32 || !args.items || !args.share || !args.context_lens ||
      args.num_seqs < 1 || args.num_seqs > kMaxSharedSeqs)
    return hipErrorInvalidValue;
  if (head_size != 128 && head_size != 64) return hipErrorInvalidValue;
  hipError_t e;
  // q of the current piece in LDS: one [num_cols][head_size + 8] slot per wavefront.
  const size_t lds = (size_t)args.heads_per_wg * args.num_cols * (head_size + 8) * sizeof(uint16_t);
  if (head_size == 128)
    e = args.block_size == 8    ? launch_decode_kernel<128, 2, kShared, 8>(args, lds, stream)
        : args.block_size == 32 ? launch_decode_kernel<128, 2, kShared, 32>(args, lds, stream)
                                : launch_decode_kernel<128, 2, kShared>(args, lds, stream);
  else
    e = args.block_size == 8    ? launch_decode_kernel<64, 2, kShared, 8>(args, lds, stream)
        : args.block_size == 32 ? launch_decode_kernel<64, 2, kShared, 32>(args, lds, stream)
                                : launch_decode_kernel<64, 2, kShared>(args, lds, stream);
  if (e != hipSuccess || args.num_wgs <= 1) return e;
  const dim3 mgrid((unsigned)args.num_wgs);
  const dim3 mblock(64 * (unsigned)args.heads_per_wg);
  if (head_size == 128) {
    hipLaunchKernelGGL((merge_kernel<128, true>), mgrid, mblock, 0, stream, args);
  } else {
    hipLaunchKernelGGL((merge_kernel<64, true>), mgrid, mblock, 0, stream, args);
  }
  return hipGetLastError();
}

// Scratch of the decode entry point that allocates nothing: a file-scope
// device array. Every GPU the library runs on holds its own copy, at its own
// address, until the process ends. Host code never passes the array's name
// to a kernel (in host code it stands for a host-side shadow, not for device
// memory): it asks the runtime for the device address once per device, with
// that device current, and keeps it.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
  static std::mutex mu;
  static std::map<int, void *> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

}  // namespace pa
