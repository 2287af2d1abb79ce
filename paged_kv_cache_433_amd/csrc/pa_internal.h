// Internal interface between the C-ABI front end (pa_api.cpp) and the HIP
// kernels (decode.hip, cache_ops.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include "../../include/pa.h"
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Sharing-aware decode: the call's work as a list of segments. A segment is
// up to 32 / group consecutive members (one sequence outside any sharing).
// Each 16-token chunk is read once, by the first member that holds it, with
// the query heads of every member that holds it too as live MFMA columns:
// member j reads its chunks from its first `own` on (the chunks before are
// those it holds in common with member j - 1, read by an earlier member),
// and they are seen by members j .. e, e being the last member after j
// whose leading shared chunks all cover it. Two ways to declare sharing feed
// this: groups with one common prefix, and a chain in which each sequence
// shares leading blocks with the one before it (a prefix tree listed depth
// first).
struct ShareItem {
  int32_t row;     // table row read for the first member's chunks < b0 (the group's first member)
  int32_t qrow;    // first member: q and output rows qrow .. qrow + ntok - 1
  int32_t ntok;    // members
  int32_t b0;      // chunks of the first member read through row `row` (0 in the chain form)
  int32_t n;       // b0 * 16
  int32_t L;       // chunks in all: what the members read themselves
  int64_t ustart;  // first unit: head groups times the chunks of all earlier segments
  int32_t eb;      // cache blocks read through row `row` (b0 = eb * block_size / 16, rounded down)
};

// Written by the plan kernel: totals of the call.
struct ShareHeader {
  int64_t units;
  int32_t items;   // segments
  int32_t empty;   // segments with no chunk (every member's context empty): the decode zeroes their rows
};

// Arguments of one decode launch, passed by value as the kernel argument.
struct DecodeArgs {
  const uint16_t *q;             // bf16 [S, q_len, Hq, D]
  const uint16_t *k_cache;       // bf16 [NB, block_size, Hkv, D]
  const uint16_t *v_cache;
  const int32_t *block_tables;   // [S, MB]
  const int32_t *context_lens;   // [S]; sharing-aware decode: the plan's member records [S][2]
  uint16_t *out;                 // bf16 [S, q_len, Hq, D]
  // [num_wgs]: the segment the workgroup's first piece ended (x, or -1), the
  // slot of its first piece (y) and, in sharing-aware decode, its first q
  // row and member count (z, w)
  int4 *merge_desc;
  float *part_ml;                // [2 * num_wgs, heads_per_wg, rec_cols, 2]: max (base 2), sum
  float *part_o;                 // [2 * num_wgs, heads_per_wg, rec_cols, D]: unnormalised output
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;                 // Hq / Hkv, <= 16
  int32_t q_len;                 // new tokens per sequence (1: decode)
  int32_t num_cols;              // q_len * group, <= kMaxDecodeCols (<= 16 when q_len == 1)
  int32_t col_groups;            // 1, or ceil(num_cols / 32) when num_cols > 32
  int32_t rec_cols;              // columns per wavefront: num_cols, or 32 when num_cols > 32
  int32_t max_blocks_per_seq;
  int32_t heads_per_wg;          // wavefronts per workgroup: KV heads (<= 4), or column groups (<= 8)
  int32_t num_head_groups;       // Hkv / heads_per_wg, or Hkv with column groups
  int32_t num_wgs;               // workgroups sharing the units evenly
  float scale_log2;              // softmax scale times log2(e)
  // The fused step only (null otherwise): each sequence's new token, bf16
  // [S, Hkv, D], attended at position n - 1 and written to its slot.
  const uint16_t *k_new;
  const uint16_t *v_new;
  // Sharing-aware decode only (null otherwise).
  const ShareItem *items;        // [num_seqs + 1]: segments, then a sentinel holding the total units
  const ShareHeader *share;
  int32_t block_size;            // tokens per cache block: 8, 16 or 32 (16 unless q_len == 1 and no sharing)
  int32_t vector_path;           // one query head per KV head: compute on the vector ALU, not matrix cores
  // Launches that stage whole-segment outputs in LDS (one column tile, not
  // 8-token blocks): outputs per wavefront (set by the launch; 0 otherwise).
  int32_t stage_slots;
  // The fused step only: 1 to write the new K/V rows to their slots, 0 when
  // a scatter launch before the decode has written them.
  int32_t write_new;
};

// Arguments of the sharing-aware plan kernel.
struct SharePlanArgs {
  const int32_t *lens;           // [S]
  const int32_t *group_starts;   // [num_groups + 1]
  const int32_t *shared_blocks;  // [num_groups]
  const int32_t *shared_prev;    // [S] in the chain form (group_starts unused then), else null
  int32_t *members;              // [S][2] out: clamped context length, chunks read through a predecessor
  ShareItem *items;
  ShareHeader *share;
  int32_t num_seqs;
  int32_t num_groups;
  int32_t max_blocks_per_seq;
  int32_t members_per_item;      // 32 / group
  int32_t group;
  int32_t num_head_groups;
  int32_t block_size;            // tokens per cache block: 8, 16 or 32
};

// Most sequences one decode call takes: the kernels read the context
// lengths through one buffer resource, whose range is a 32-bit byte count.
constexpr int32_t kMaxDecodeSeqs = 1 << 28;

// Most (new token, query head) columns one wavefront takes for a KV head
// (four MFMA tiles of 16); past them a workgroup serves one KV head with a
// wavefront per 32 columns.
constexpr int32_t kMaxNarrowCols = 64;

// Most (new token, query head) columns per KV head a decode launch takes:
// 8 column groups of 32, one wavefront each.
constexpr int32_t kMaxDecodeCols = 256;

// How a decode call is split and what scratch it needs (host only).
struct DecodePlan {
  int32_t heads_per_wg;          // wavefronts per workgroup
  int32_t num_head_groups;
  int32_t col_groups;
  int32_t rec_cols;
  int32_t num_wgs;
  size_t desc_bytes;             // offset of part_ml
  size_t ml_bytes;
  size_t o_bytes;
  size_t total_bytes;            // 0 when num_wgs == 1 (nothing is ever cut)
};

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_size, int32_t max_chunks_per_seq, int32_t q_len);

hipError_t launch_decode(const DecodeArgs &args, int32_t head_size, hipStream_t stream);

// Whole-segment outputs a wavefront of a one-tile decode launch stages in
// LDS (0 with 8-token blocks or more than 16 columns); `new_rows`: the
// decode step writing its new rows, whose slots take part of the room.
int32_t decode_stage_slots(int32_t num_cols, int32_t head_size, int32_t block_size, bool new_rows);

// The new tokens of a decode step to their slots, found from the tables and
// context lengths as the fused step finds them (cache_ops.hip).
hipError_t launch_step_scatter(const uint16_t *k, const uint16_t *v, const int32_t *tables, const int32_t *lens,
                               uint16_t *k_cache, uint16_t *v_cache, int32_t num_seqs, int32_t row_elems,
                               int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks,
                               hipStream_t stream);

// Bytes of the static device scratch of pa_decode_noalloc. It covers every
// single-token decode the default split can produce: at most 1024
// workgroups x KV heads per workgroup, 16 columns each, head size 128, two
// partial records per (workgroup, head, column): merge records 16 KiB,
// max/sum 256 KiB, outputs 16 MiB.
constexpr size_t kNoAllocScratchBytes = ((size_t)16 << 20) + ((size_t)512 << 10);
static_assert(kNoAllocScratchBytes == PA_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

// Device address of that scratch on the current device (looked up once per
// device and kept).
hipError_t noalloc_scratch(void **ptr);

// Largest batch the sharing-aware plan kernel takes (it keeps per-sequence
// and per-group state in LDS).
constexpr int32_t kMaxSharedSeqs = 4096;

// The plan of a sharing-aware call: its segments (plan.items, plan.share)
// and member records (plan.members), from the context lengths and the
// declaration alone.
hipError_t launch_share_plan(const SharePlanArgs &plan, hipStream_t stream);

// Decode and merge of a sharing-aware call on a plan: args.items, args.share
// and, in place of the context lengths, args.context_lens = the plan's
// member records. args.num_cols is the segment width (members_per_item *
// group), args.q_len is 1.
hipError_t launch_decode_planned(const DecodeArgs &args, int32_t head_size, hipStream_t stream);

hipError_t launch_reshape_and_cache(const uint16_t *k, const uint16_t *v, const int64_t *slots,
                                    uint16_t *k_cache, uint16_t *v_cache, int32_t num_tokens,
                                    int32_t row_elems, int64_t num_slots, hipStream_t stream);

hipError_t launch_copy_blocks(uint16_t *k_cache, uint16_t *v_cache, const int64_t *pairs,
                              int32_t num_pairs, int64_t block_elems, int64_t num_blocks,
                              hipStream_t stream);

hipError_t launch_swap_blocks(const uint16_t *from_k, const uint16_t *from_v, int64_t from_blocks, uint16_t *to_k,
                              uint16_t *to_v, int64_t to_blocks, const int64_t *pairs, int32_t num_pairs,
                              int64_t block_elems, hipStream_t stream);

hipError_t launch_probe_copy(void *dst, const void *src, size_t bytes, hipStream_t stream);

// Workgroups of the read probe (256 threads each); its sink holds one
// 32-bit word per thread.
constexpr unsigned kProbeReadBlocks = 256 * 32;
hipError_t launch_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

}  // namespace pa
