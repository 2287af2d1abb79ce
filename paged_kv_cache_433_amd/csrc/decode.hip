// Paged decode attention for CDNA4 (gfx950).
//
// What is computed: for each sequence, one new query token per query head
// attends over the sequence's cached K/V. The cache sits in 16-token physical
// blocks that the sequence's block table maps from logical blocks ("vLLM:
// Anatomy and Mechanisms of High-Throughput LLM Inference", section
// "Block-Level Management"; decode semantics from "Inside vLLM: Anatomy of a
// High-Throughput LLM Inference System", section "Scheduler").
//
// Work split. One wavefront (64 lanes, one workgroup) owns one (sequence,
// KV head, partition) item: a run of `part_blocks` blocks. It serves every
// query head of the KV head's group (G <= 16), so each K/V byte is read
// from HBM once for the whole group. A sequence that fits one partition
// writes its bf16 output directly. Longer ones write fp32 partials (running
// max, sum, unnormalised output) that are merged with log-sum-exp weights:
// by the last partition to finish (an epoch-tagged counter per sequence and
// KV head in the workspace), or by a separate merge kernel when there are
// many partitions.
//
// Inner loop, per pair of blocks (32 tokens), all on matrix cores:
//   * QK^T on v_mfma_f32_16x16x32_bf16: rows are the 16 tokens of a block,
//     columns the 16 query-head slots, and the reduction runs over head_size.
//     Lane (c, grp) (c = lane % 16, grp = lane / 16) loads, for MFMA step
//     j, the 16 bytes at head dims 32*j + 8*grp of token c's row, so each
//     load instruction reads a contiguous 64-byte piece of 16 token rows. The
//     sum over head_size is order-free, so q is loaded with the same mapping.
//     The result gives lane (c, grp) the logits of query head c for tokens
//     4*grp..4*grp+3.
//   * V must be transposed (tokens along registers) before it can be a
//     matrix operand of P*V. The transpose is itself an MFMA: multiplying the
//     V rows by a one-hot 16x16 selector (v_mfma_f32_16x16x16_bf16) lands,
//     in lane (c, grp), V[4*grp + r][d(c)] for r = 0..3. That is exactly the
//     token set whose probabilities the same lane holds. The values are exact
//     bf16, so their upper halves repack into an operand with v_perm.
//   * P*V on v_mfma_f32_16x16x32_bf16, with P split into two bf16 terms
//     (high part plus rounding residue) so the product keeps about 16
//     significant bits of P. The accumulator layout leaves lane (c, grp)
//     with output dims 32*j + 8*grp .. +7 of query head c for every j, so
//     results leave as 16-byte stores.
// Online softmax works in base 2 (logits prescaled by scale*log2 e, hardware
// exp2). Row maxima are shared by the four lanes of a head with two
// cross-lane exchanges per pair of blocks; row sums stay lane-partial until
// the end.
//
// Tokens past the context length are masked by a select on the logit, and
// their V rows are zeroed, so stale data in the tail of the last block
// (even NaN) cannot reach the output. Block ids are clamped to the pool, and
// no table entry past the last used block is read.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

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

constexpr int kBlock = 16;
constexpr uint32_t kBf16One = 0x3F80u;

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

// Count this partition as finished; return how many of this call's
// partitions have finished, this one included. A counter word holds the
// call's epoch in its upper half and the count in its lower half, so a word
// left over from another call (or never initialised) reads as zero
// arrivals: the first arrival of this call replaces it. Lock-free: every
// failed compare-and-swap means another arrival succeeded, so at most one
// retry per partition.
__device__ __forceinline__ int arrive(unsigned long long *ctr, uint32_t epoch) {
  unsigned long long old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (true) {
    const unsigned long long want = (uint32_t)(old >> 32) == epoch
                                        ? old + 1ull
                                        : (((unsigned long long)epoch << 32) | 1ull);
    const unsigned long long seen = atomicCAS(ctr, old, want);
    if (seen == old) return (int)(uint32_t)want;
    old = seen;
  }
}

template <int D>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeArgs a) {
  constexpr int NJ = D / 32;  // MFMA steps over head_size; 16-byte loads per lane per row
  static_assert(NJ >= 1 && D % 32 == 0, "head_size must be a multiple of 32");

  const int lane = threadIdx.x;
  const int c = lane & 15;
  const int grp = lane >> 4;
  const int sg = blockIdx.x;
  const int s = sg / a.num_kv_heads;
  const int g = sg - s * a.num_kv_heads;
  const int part = blockIdx.y;

  int n = a.context_lens[s];
  n = n < 0 ? 0 : (n > a.max_blocks_per_seq * kBlock ? a.max_blocks_per_seq * kBlock : n);
  const int nblk = (n + kBlock - 1) / kBlock;
  const int b_begin = part * a.part_blocks;
  const bool head_ok = c < a.group;
  const int head = g * a.group + (head_ok ? c : 0);
  uint16_t *out_row = a.out + ((size_t)s * a.num_q_heads + head) * D + grp * 8;

  if (n == 0) {  // nothing cached: zero output, written once
    if (part == 0 && head_ok) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) *reinterpret_cast<u32x4_t *>(out_row + 32 * j) = u32x4_t{0, 0, 0, 0};
    }
    return;
  }
  if (b_begin >= nblk) return;
  const int b_end = min(nblk, b_begin + a.part_blocks);
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;

  // q of query head c, with the head-dim mapping this lane uses for K rows.
  u32x4_t qv[NJ];
  {
    const uint16_t *q_row = a.q + ((size_t)s * a.num_q_heads + head) * D + grp * 8;
#pragma unroll
    for (int j = 0; j < NJ; ++j) qv[j] = head_ok ? load16(q_row + 32 * j) : u32x4_t{0, 0, 0, 0};
  }

  // Physical ids of this partition's blocks, one per lane, clamped to the pool.
  int my_blk = 0;
  if (lane < b_end - b_begin) {
    my_blk = a.block_tables[(size_t)s * a.max_blocks_per_seq + b_begin + lane];
    if (my_blk < 0 || (int64_t)my_blk >= a.num_blocks) my_blk = 0;
  }

  const size_t tok_stride = (size_t)a.num_kv_heads * D;  // elements between tokens
  const size_t blk_stride = tok_stride * kBlock;
  const size_t lane_off = (size_t)c * tok_stride + (size_t)g * D + grp * 8;
  const uint16_t *kbase = a.k_cache + lane_off;
  const uint16_t *vbase = a.v_cache + lane_off;

  // One-hot selector: column n of the 16x16 selector picks operand slot
  // (group n/4, element n%4), i.e. lane (c, grp) holds 1.0 in element c%4
  // iff grp == c/4.
  u32x2_t sel = {0u, 0u};
  if (grp == (c >> 2)) {
    const uint32_t word = (c & 1) ? (kBf16One << 16) : kBf16One;
    if (c & 2) sel.y = word; else sel.x = word;
  }

  float m_run = -INFINITY;  // running max of base-2 logits, head c
  float l_run = 0.f;        // this lane's share of the running sum
  f32x4_t acc[2 * NJ];
#pragma unroll
  for (int t = 0; t < 2 * NJ; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  for (int b = b_begin; b < b_end; b += 2) {
    const int i0 = b - b_begin;
    const bool has1 = b + 1 < b_end;
    const int blk0 = __builtin_amdgcn_readlane(my_blk, i0);
    const int blk1 = __builtin_amdgcn_readlane(my_blk, i0 + 1);
    const uint16_t *k0 = kbase + (size_t)blk0 * blk_stride;
    const uint16_t *v0 = vbase + (size_t)blk0 * blk_stride;
    const uint16_t *k1 = kbase + (size_t)blk1 * blk_stride;
    const uint16_t *v1 = vbase + (size_t)blk1 * blk_stride;

    u32x4_t K0[NJ], K1[NJ], V0[NJ], V1[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) K0[j] = load16(k0 + 32 * j);
#pragma unroll
    for (int j = 0; j < NJ; ++j) V0[j] = load16(v0 + 32 * j);
    if (has1) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) K1[j] = load16(k1 + 32 * j);
#pragma unroll
      for (int j = 0; j < NJ; ++j) V1[j] = load16(v1 + 32 * j);
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) K1[j] = V1[j] = u32x4_t{0, 0, 0, 0};
    }

    // logits: lane holds tokens 4*grp + r of each block, query head c
    f32x4_t s0 = zero4, s1 = zero4;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      s0 = mfma32(K0[j], qv[j], s0);
      s1 = mfma32(K1[j], qv[j], s1);
    }
    const int pos0 = b * kBlock + grp * 4;
    float z[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = (pos0 + r < n) ? s0[r] * a.scale_log2 : -INFINITY;
      z[4 + r] = (pos0 + kBlock + r < n) ? s1[r] * a.scale_log2 : -INFINITY;
    }
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);  // finite: token b*16 is always < n
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    // P = P_hi + P_lo, both bf16: the pair carries ~16 significant bits, so
    // rounding P does not get amplified when the V terms nearly cancel.
    u32x4_t pb_hi, pb_lo;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = fast_exp2(z[2 * i] - m_new);
      const float p1 = fast_exp2(z[2 * i + 1] - m_new);
      const uint32_t hi = to_bf16x2(p0, p1);
      pb_hi[i] = hi;
      pb_lo[i] = to_bf16x2(p0 - bf16_lo(hi), p1 - bf16_hi(hi));
      psum += p0 + p1;
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t = 0; t < 2 * NJ; ++t) acc[t] *= alpha;

    // V rows of tokens at or past n must not reach the sum, even as NaN * 0.
    if ((b + 2) * kBlock > n) {
      if (b * kBlock + c >= n) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) V0[j] = u32x4_t{0, 0, 0, 0};
      }
      if ((b + 1) * kBlock + c >= n) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) V1[j] = u32x4_t{0, 0, 0, 0};
      }
    }

#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4_t t0 = mfma16(u32x2_t{V0[j][2 * h], V0[j][2 * h + 1]}, sel, zero4);
        const f32x4_t t1 = mfma16(u32x2_t{V1[j][2 * h], V1[j][2 * h + 1]}, sel, zero4);
        const u32x4_t av = {pack_hi(t0[0], t0[1]), pack_hi(t0[2], t0[3]), pack_hi(t1[0], t1[1]),
                            pack_hi(t1[2], t1[3])};
        acc[2 * j + h] = mfma32(av, pb_hi, acc[2 * j + h]);
        acc[2 * j + h] = mfma32(av, pb_lo, acc[2 * j + h]);
      }
    }
  }

  float l = l_run + __shfl_xor(l_run, 16);
  l += __shfl_xor(l, 32);

  if (nparts == 1) {
    if (head_ok) store_out<NJ>(out_row, acc, 1.f / l);
    return;
  }

  // Partial result of this partition.
  const size_t prow = ((size_t)s * a.num_q_heads + head) * a.max_parts + part;
  if (head_ok) {
    float *po = a.part_o + prow * D + grp * 8;
#pragma unroll
    for (int t = 0; t < 2 * NJ; ++t) *reinterpret_cast<f32x4_t *>(po + 32 * (t >> 1) + 4 * (t & 1)) = acc[t];
    if (grp == 0) *reinterpret_cast<f32x2_t *>(a.part_ml + prow * 2) = f32x2_t{m_run, l};
  }
  if (!a.fused_merge) return;

  // The last partition of this (sequence, KV head) to finish merges them all.
  __threadfence();
  int arrived = 0;
  if (lane == 0) arrived = arrive(a.counters + sg, a.epoch);
  arrived = __shfl(arrived, 0);
  if (arrived != nparts) return;
  __threadfence();
  if (!head_ok) return;

  const size_t base = ((size_t)s * a.num_q_heads + head) * a.max_parts;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.part_ml[(base + p) * 2]);
  float L = 0.f;
  f32x4_t o[2 * NJ];
#pragma unroll
  for (int t = 0; t < 2 * NJ; ++t) o[t] = zero4;
  for (int p = 0; p < nparts; ++p) {
    const f32x2_t ml = *reinterpret_cast<const f32x2_t *>(a.part_ml + (base + p) * 2);
    const float w = fast_exp2(ml[0] - M);
    L += w * ml[1];
    const float *po = a.part_o + (base + p) * D + grp * 8;
#pragma unroll
    for (int t = 0; t < 2 * NJ; ++t)
      o[t] += w * *reinterpret_cast<const f32x4_t *>(po + 32 * (t >> 1) + 4 * (t & 1));
  }
  store_out<NJ>(out_row, o, 1.f / L);
}

// Separate log-sum-exp merge for calls with many partitions per sequence:
// one wavefront per (sequence, query head); lane i owns dims [i*D/64, ...).
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(const DecodeArgs a) {
  constexpr int PL = D / 64;  // dims per lane: 1 or 2
  const int lane = threadIdx.x;
  const int s = blockIdx.x / a.num_q_heads;
  const int h = blockIdx.x - s * a.num_q_heads;
  int n = a.context_lens[s];
  n = n < 0 ? 0 : (n > a.max_blocks_per_seq * kBlock ? a.max_blocks_per_seq * kBlock : n);
  const int nblk = (n + kBlock - 1) / kBlock;
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;
  if (nparts <= 1) return;  // written by the decode kernel itself

  const size_t base = ((size_t)s * a.num_q_heads + h) * a.max_parts;
  float M = -INFINITY;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, a.part_ml[(base + p) * 2]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  float L = 0.f;
  float o[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) o[i] = 0.f;
#pragma unroll 4
  for (int p = 0; p < nparts; ++p) {
    const f32x2_t ml = *reinterpret_cast<const f32x2_t *>(a.part_ml + (base + p) * 2);
    const float w = fast_exp2(ml[0] - M);
    L += w * ml[1];
    const float *po = a.part_o + (base + p) * D + lane * PL;
#pragma unroll
    for (int i = 0; i < PL; ++i) o[i] += w * po[i];
  }
  const float inv = 1.f / L;
  uint16_t *dst = a.out + ((size_t)s * a.num_q_heads + h) * D + lane * PL;
  if constexpr (PL == 2) {
    *reinterpret_cast<uint32_t *>(dst) = to_bf16x2(o[0] * inv, o[1] * inv);
  } else {
    dst[0] = (uint16_t)(to_bf16x2(o[0] * inv, 0.f) & 0xFFFFu);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &args, int32_t head_size, hipStream_t stream) {
  const dim3 grid((unsigned)args.num_seqs * (unsigned)args.num_kv_heads, (unsigned)args.max_parts);
  const dim3 block(64);
  if (head_size == 128) {
    hipLaunchKernelGGL(decode_kernel<128>, grid, block, 0, stream, args);
  } else if (head_size == 64) {
    hipLaunchKernelGGL(decode_kernel<64>, grid, block, 0, stream, args);
  } else {
    return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || args.max_parts <= 1 || args.fused_merge) return err;
  const dim3 mgrid((unsigned)args.num_seqs * (unsigned)args.num_q_heads);
  if (head_size == 128) {
    hipLaunchKernelGGL(merge_kernel<128>, mgrid, block, 0, stream, args);
  } else {
    hipLaunchKernelGGL(merge_kernel<64>, mgrid, block, 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace pa
