// Paged decode attention for CDNA4 (gfx950).
//
// What is computed: for each sequence, one new query token per query head
// attends over the sequence's cached K/V. The cache sits in 16-token physical
// blocks that the sequence's block table maps from logical blocks ("vLLM:
// Anatomy and Mechanisms of High-Throughput LLM Inference", section
// "Block-Level Management"; decode semantics from "Inside vLLM: Anatomy of a
// High-Throughput LLM Inference System", section "Scheduler").
//
// Work split (balanced). KV heads form groups of HG heads (HG = largest
// divisor of num_kv_heads that is <= 8). A "unit" is one physical block of
// one sequence for one head group; a "segment" is all units of one
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
// Inner loop, per block (16 tokens), on matrix cores:
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
// Tokens past the context length are masked by a select on the logit and
// their V rows are zeroed, so stale data in the tail of the last block (even
// NaN) cannot reach the output. Block ids are clamped to the pool, and no
// table entry past a sequence's last used block is read.

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

__device__ __forceinline__ int clamp_len(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }

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

// Attention of one wavefront's query heads over blocks [b_begin, b_end) of
// sequence s, KV head g (n tokens cached). Returns, for query head c of the
// group (lane (c, grp)), the running max m_run (base 2), this lane's share
// of the sum of weights l_part, and the unnormalised output in acc.
template <int D>
__device__ __forceinline__ void attend_blocks(const DecodeArgs &a, int s, int g, int b_begin,
                                              int b_end, int n, const u32x4_t (&qv)[D / 32],
                                              float &m_run, float &l_part,
                                              f32x4_t (&acc)[2 * (D / 32)]) {
  constexpr int NJ = D / 32;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int grp = lane >> 4;

  const size_t tok_stride = (size_t)a.num_kv_heads * D;  // elements between tokens
  const size_t blk_stride = tok_stride * kBlock;
  const size_t lane_off = (size_t)c * tok_stride + (size_t)g * D + grp * 8;
  const uint16_t *kbase = a.k_cache + lane_off;
  const uint16_t *vbase = a.v_cache + lane_off;
  const int32_t *table = a.block_tables + (size_t)s * a.max_blocks_per_seq;

  // One-hot selector: lane (c, grp) holds 1.0 in element c%4 iff grp == c/4.
  u32x2_t sel = {0u, 0u};
  if (grp == (c >> 2)) {
    const uint32_t word = (c & 1) ? (kBf16One << 16) : kBf16One;
    if (c & 2) sel.y = word; else sel.x = word;
  }
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int chunk = b_begin; chunk < b_end; chunk += 64) {
    const int cnt = min(64, b_end - chunk);
    // Physical ids of up to 64 blocks, one per lane, clamped to the pool.
    int my_blk = 0;
    if (lane < cnt) {
      my_blk = table[chunk + lane];
      if (my_blk < 0 || (int64_t)my_blk >= a.num_blocks) my_blk = 0;
    }
    for (int i = 0; i < cnt; ++i) {
      const int b = chunk + i;
      const int blk = __builtin_amdgcn_readlane(my_blk, i);
      const uint16_t *kp = kbase + (size_t)blk * blk_stride;
      const uint16_t *vp = vbase + (size_t)blk * blk_stride;
      u32x4_t K[NJ], V[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) K[j] = load16(kp + 32 * j);
#pragma unroll
      for (int j = 0; j < NJ; ++j) V[j] = load16(vp + 32 * j);

      f32x4_t sc = zero4;
#pragma unroll
      for (int j = 0; j < NJ; ++j) sc = mfma32(K[j], qv[j], sc);
      const int pos0 = b * kBlock + grp * 4;
      float z[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) z[r] = (pos0 + r < n) ? sc[r] * a.scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);  // finite: token b*16 is always < n
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;

      // P = P_hi + P_lo, both bf16.
      const float p0 = fast_exp2(z[0] - m_new), p1 = fast_exp2(z[1] - m_new);
      const float p2 = fast_exp2(z[2] - m_new), p3 = fast_exp2(z[3] - m_new);
      const uint32_t h01 = to_bf16x2(p0, p1), h23 = to_bf16x2(p2, p3);
      const u32x2_t pb_hi = {h01, h23};
      const u32x2_t pb_lo = {to_bf16x2(p0 - bf16_lo(h01), p1 - bf16_hi(h01)),
                             to_bf16x2(p2 - bf16_lo(h23), p3 - bf16_hi(h23))};
      l_part = l_part * alpha + ((p0 + p1) + (p2 + p3));
#pragma unroll
      for (int t = 0; t < 2 * NJ; ++t) acc[t] *= alpha;

      // V rows of tokens at or past n must not reach the sum, even as NaN * 0.
      if (b * kBlock + c >= n) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) V[j] = u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4_t t = mfma16(u32x2_t{V[j][2 * h], V[j][2 * h + 1]}, sel, zero4);
          const u32x2_t av = {pack_hi(t[0], t[1]), pack_hi(t[2], t[3])};
          acc[2 * j + h] = mfma16(av, pb_hi, acc[2 * j + h]);
          acc[2 * j + h] = mfma16(av, pb_lo, acc[2 * j + h]);
        }
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
void decode_kernel(const DecodeArgs a) {
  constexpr int NJ = D / 32;
  static_assert(NJ >= 1 && D % 32 == 0, "head_size must be a multiple of 32");
  __shared__ long long red[8];
  __shared__ int found_seq;
  __shared__ long long found_prefix;

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 15;
  const int grp = lane >> 4;
  const int w = blockIdx.x;
  const int S = a.num_seqs;
  const int NG = a.num_head_groups;
  const int HG = a.heads_per_wg;
  const int cap = a.max_blocks_per_seq * kBlock;
  const long long W = a.num_wgs;

  // Pass 1: total units; zero rows (and "no merge" records) for empty sequences.
  long long mine = 0;
  for (int s = tid; s < S; s += nthr) {
    const int n = clamp_len(a.context_lens[s], cap);
    mine += (n + kBlock - 1) / kBlock;
    if (n == 0 && s % a.num_wgs == w) {
      u32x4_t *row = reinterpret_cast<u32x4_t *>(a.out + (size_t)s * a.num_q_heads * D);
      for (int i = 0; i < a.num_q_heads * D / 8; ++i) row[i] = u32x4_t{0, 0, 0, 0};
      if (a.merge_desc)
        for (int hg = 0; hg < NG; ++hg) a.merge_desc[(size_t)s * NG + hg] = int2{-1, -1};
    }
  }
  const long long U = wg_sum(mine, red, wave, lane, nthr >> 6) * NG;
  const long long E = U < W ? U : W;  // workgroups that get units
  if (w >= E) return;
  const long long lo = range_lo(w, U, E);
  const long long hi = range_lo(w + 1, U, E);

  // Pass 2: the sequence whose units hold `lo` (block scan over the lengths).
  if (tid == 0) found_seq = -1;
  long long before = 0;  // blocks of all sequences preceding this chunk
  for (int base = 0; base < S; base += nthr) {
    const int s = base + tid;
    const long long L = s < S ? (clamp_len(a.context_lens[s], cap) + kBlock - 1) / kBlock : 0;
    long long incl = L;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    __syncthreads();
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    long long pre = before;
    long long chunk_total = 0;
    for (int i = 0; i < (nthr >> 6); ++i) {
      if (i < wave) pre += red[i];
      chunk_total += red[i];
    }
    const long long excl = pre + incl - L;
    if (L > 0 && excl * NG <= lo && lo < (excl + L) * NG) {
      found_seq = s;
      found_prefix = excl;
    }
    __syncthreads();
    if (found_seq >= 0) break;
    before += chunk_total;
  }

  if (found_seq < 0) return;  // only if the lengths changed during the call

  // Walk the range, piece by piece; every wavefront takes KV head
  // hg*HG + wave of each piece.
  int s = found_seq;
  long long seg_base = found_prefix * NG;  // first unit of sequence s
  int n = clamp_len(a.context_lens[s], cap);
  int L = (n + kBlock - 1) / kBlock;
  int hg = (int)((lo - seg_base) / L);
  int off = (int)((lo - seg_base) % L);
  long long u = lo;
  bool first = true;
  const bool head_ok = c < a.group;

  while (u < hi) {
    const long long seg_start = seg_base + (long long)hg * L;
    const int piece = (int)min((long long)(L - off), hi - u);
    const int g = hg * HG + wave;
    const int head = g * a.group + (head_ok ? c : 0);

    u32x4_t qv[NJ];
    {
      const uint16_t *q_row = a.q + ((size_t)s * a.num_q_heads + head) * D + grp * 8;
#pragma unroll
      for (int j = 0; j < NJ; ++j) qv[j] = head_ok ? load16(q_row + 32 * j) : u32x4_t{0, 0, 0, 0};
    }
    float m_run = -INFINITY, l_part = 0.f;
    f32x4_t acc[2 * NJ];
#pragma unroll
    for (int t = 0; t < 2 * NJ; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    attend_blocks<D>(a, s, g, off, off + piece, n, qv, m_run, l_part, acc);
    float l = l_part + __shfl_xor(l_part, 16);
    l += __shfl_xor(l, 32);

    const bool whole = off == 0 && piece == L;
    const bool ends_here = off + piece == L;
    if (whole) {
      if (head_ok) store_out<NJ>(a.out + ((size_t)s * a.num_q_heads + head) * D + grp * 8, acc, 1.f / l);
    } else {
      const int slot = first ? 0 : 1;
      const size_t row = (((size_t)w * 2 + slot) * HG + wave) * a.group + c;
      if (head_ok) {
        float *po = a.part_o + row * D + grp * 8;
#pragma unroll
        for (int t = 0; t < 2 * NJ; ++t)
          *reinterpret_cast<f32x4_t *>(po + 32 * (t >> 1) + 4 * (t & 1)) = acc[t];
        if (grp == 0) *reinterpret_cast<f32x2_t *>(a.part_ml + row * 2) = f32x2_t{m_run, l};
      }
    }
    if (ends_here && tid == 0 && a.merge_desc) {
      int2 d = {-1, -1};
      if (!whole) {  // the segment began in an earlier workgroup: record its pieces
        const int w0 = owner_of(seg_start, U, E);
        const int slot0 = range_lo(w0, U, E) < seg_start ? 1 : 0;
        d = int2{w0 * 2 + slot0, w};
      }
      a.merge_desc[(size_t)s * NG + hg] = d;
    }

    first = false;
    u += piece;
    off += piece;
    if (off == L) {
      off = 0;
      if (++hg == NG && u < hi) {
        hg = 0;
        seg_base += (long long)NG * L;
        do {  // units remain, so a non-empty sequence follows
          ++s;
          n = s < S ? clamp_len(a.context_lens[s], cap) : 0;
          L = (n + kBlock - 1) / kBlock;
        } while (L == 0 && s < S);
        if (s >= S) break;  // only if the lengths changed during the call
      }
    }
  }
}

// Log-sum-exp merge of the pieces of segments cut by workgroup boundaries.
// Grid: (num_seqs * num_head_groups, heads_per_wg); one wavefront per query
// head of the group; lane i owns head dims [i*D/64, (i+1)*D/64).
template <int D>
__global__ __launch_bounds__(1024) void merge_kernel(const DecodeArgs a) {
  constexpr int PL = D / 64;  // dims per lane: 1 or 2
  const int seg = blockIdx.x;
  const int2 d = a.merge_desc[seg];
  if (d.x < 0) return;
  const int lane = threadIdx.x & 63;
  const int c = threadIdx.x >> 6;            // query head within the KV head's group
  const int wave = blockIdx.y;               // KV head within the head group
  const int s = seg / a.num_head_groups;
  const int hg = seg - s * a.num_head_groups;
  const int g = hg * a.heads_per_wg + wave;
  const int w0 = d.x >> 1, w1 = d.y;
  const int HG = a.heads_per_wg;

  auto rec_row = [&](int w) -> size_t {
    const int rec = w == w0 ? d.x : 2 * w;
    return ((size_t)rec * HG + wave) * a.group + c;
  };
  // Pieces: slot d.x & 1 of workgroup w0, then the first slot of every
  // workgroup up to w1 (whose ranges all lie inside the segment).
  float M = -INFINITY;
  for (int w = w0; w <= w1; ++w) M = fmaxf(M, a.part_ml[rec_row(w) * 2]);
  float Lsum = 0.f;
  float o[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) o[i] = 0.f;
#pragma unroll 4
  for (int w = w0; w <= w1; ++w) {
    const size_t r = rec_row(w);
    const f32x2_t ml = *reinterpret_cast<const f32x2_t *>(a.part_ml + r * 2);
    const float wt = fast_exp2(ml[0] - M);
    Lsum += wt * ml[1];
    const float *po = a.part_o + r * D + lane * PL;
#pragma unroll
    for (int i = 0; i < PL; ++i) o[i] += wt * po[i];
  }
  const float inv = 1.f / Lsum;
  uint16_t *dst = a.out + ((size_t)s * a.num_q_heads + (size_t)g * a.group + c) * D + lane * PL;
  if constexpr (PL == 2) {
    *reinterpret_cast<uint32_t *>(dst) = to_bf16x2(o[0] * inv, o[1] * inv);
  } else {
    dst[0] = (uint16_t)(to_bf16x2(o[0] * inv, 0.f) & 0xFFFFu);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &args, int32_t head_size, hipStream_t stream) {
  const dim3 grid((unsigned)args.num_wgs);
  const dim3 block(64 * (unsigned)args.heads_per_wg);
  if (head_size == 128) {
    hipLaunchKernelGGL(decode_kernel<128>, grid, block, 0, stream, args);
  } else if (head_size == 64) {
    hipLaunchKernelGGL(decode_kernel<64>, grid, block, 0, stream, args);
  } else {
    return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || args.num_wgs <= 1) return err;
  const dim3 mgrid((unsigned)args.num_seqs * (unsigned)args.num_head_groups,
                   (unsigned)args.heads_per_wg);
  const dim3 mblock(64 * (unsigned)args.group);
  if (head_size == 128) {
    hipLaunchKernelGGL(merge_kernel<128>, mgrid, mblock, 0, stream, args);
  } else {
    hipLaunchKernelGGL(merge_kernel<64>, mgrid, mblock, 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace pa
