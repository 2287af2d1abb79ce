// Internal interface between the C-ABI front end (pa_api.cpp) and the HIP
// kernels (decode.hip, cache_ops.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Arguments of one decode launch, passed by value as the kernel argument.
struct DecodeArgs {
  const uint16_t *q;             // bf16 [S, Hq, D]
  const uint16_t *k_cache;       // bf16 [NB, 16, Hkv, D]
  const uint16_t *v_cache;
  const int32_t *block_tables;   // [S, MB]
  const int32_t *context_lens;   // [S]
  uint16_t *out;                 // bf16 [S, Hq, D]
  unsigned long long *counters;  // [S * Hkv] epoch-tagged completion counters
  float *part_ml;                // [S, Hq, max_parts, 2]: running max (base 2), sum
  float *part_o;                 // [S, Hq, max_parts, D]: unnormalised output
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;                 // Hq / Hkv, <= 16
  int32_t max_blocks_per_seq;
  int32_t part_blocks;           // blocks per partition: even, 2..64
  int32_t max_parts;             // ceil(max_blocks_per_seq / part_blocks)
  int32_t fused_merge;           // 1: the last partition of a (seq, KV head) merges
  float scale_log2;              // softmax scale times log2(e)
  uint32_t epoch;                // nonzero, distinct for consecutive calls
};

// How a decode call is split and what scratch it needs (host only).
struct DecodePlan {
  int32_t part_blocks;
  int32_t max_parts;
  int32_t fused_merge;
  size_t counters_bytes;         // 8 bytes per (sequence, KV head); offset of part_ml
  size_t ml_bytes;
  size_t o_bytes;
  size_t total_bytes;            // 0 when max_parts == 1
};

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_size, int32_t max_blocks_per_seq);

hipError_t launch_decode(const DecodeArgs &args, int32_t head_size, hipStream_t stream);

hipError_t launch_reshape_and_cache(const uint16_t *k, const uint16_t *v, const int64_t *slots,
                                    uint16_t *k_cache, uint16_t *v_cache, int32_t num_tokens,
                                    int32_t row_elems, int64_t num_slots, hipStream_t stream);

hipError_t launch_copy_blocks(uint16_t *k_cache, uint16_t *v_cache, const int64_t *pairs,
                              int32_t num_pairs, int64_t block_elems, int64_t num_blocks,
                              hipStream_t stream);

hipError_t launch_probe_copy(void *dst, const void *src, size_t bytes, hipStream_t stream);

}  // namespace pa
