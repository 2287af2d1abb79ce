// Cache maintenance kernels for CDNA4 (gfx950): slot scatter, copy-on-write
// block copy, and a plain 16-byte copy used for measurement.
//
// Both cache kernels are bit copies. They only move 16-byte vectors, and
// every index taken from device memory is range-checked: a slot or block
// outside the pool is skipped, never dereferenced.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One workgroup per new token. The token's K row and V row (num_kv_heads *
// head_size elements each) go to physical slot slot_mapping[t]: offset
// slot % block_size of block slot / block_size ("vLLM: Anatomy and Mechanisms of
// High-Throughput LLM Inference", section "Block-Level Management": a block
// from the free pool receives the tokens of its logical block as they come).
// In the [num_blocks, block_size, Hkv, D] layout a slot's row is contiguous and
// starts at element slot * row_elems.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const int64_t *__restrict__ slots,
    uint16_t *__restrict__ k_cache, uint16_t *__restrict__ v_cache, int32_t row_elems,
    int64_t num_slots) {
  const int t = blockIdx.x;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int vecs = row_elems / 8;
  const u32x4_t *ks = reinterpret_cast<const u32x4_t *>(k + (size_t)t * row_elems);
  const u32x4_t *vs = reinterpret_cast<const u32x4_t *>(v + (size_t)t * row_elems);
  u32x4_t *kd = reinterpret_cast<u32x4_t *>(k_cache + (size_t)slot * row_elems);
  u32x4_t *vd = reinterpret_cast<u32x4_t *>(v_cache + (size_t)slot * row_elems);
  for (int i = threadIdx.x; i < vecs; i += blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

// The scatter of a decode step's new tokens, each to the slot of its
// position n - 1 (n = the sequence's context length clamped to 0 ..
// max_blocks_per_seq * block_size): row (n - 1) % block_size of the block
// its table names there ("vLLM: Anatomy and Mechanisms", section
// "Block-Level Management"). Empty sequences and table entries outside the
// pool write nothing. The same slots, clamps and skips as the fused step's
// own writes. Workgroups take sequences in turn; threads take 16-byte
// vectors of the token row (all KV heads).
__global__ __launch_bounds__(256) void step_scatter_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const int32_t *__restrict__ tables,
    const int32_t *__restrict__ lens, uint16_t *__restrict__ k_cache, uint16_t *__restrict__ v_cache,
    int32_t num_seqs, int32_t row_elems, int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks) {
  const int cap = max_blocks_per_seq * block_size;
  const int vecs = row_elems / 8;
  for (int s = blockIdx.x; s < num_seqs; s += gridDim.x) {
    const int len = lens[s];
    const int n = len < 0 ? 0 : (len > cap ? cap : len);
    if (n == 0) continue;
    const int pos = n - 1;
    const int id = tables[(size_t)s * max_blocks_per_seq + pos / block_size];
    if (id < 0 || id >= num_blocks) continue;
    const size_t dst = ((size_t)id * block_size + pos % block_size) * row_elems;
    const u32x4_t *ks = reinterpret_cast<const u32x4_t *>(k + (size_t)s * row_elems);
    const u32x4_t *vs = reinterpret_cast<const u32x4_t *>(v + (size_t)s * row_elems);
    u32x4_t *kd = reinterpret_cast<u32x4_t *>(k_cache + dst);
    u32x4_t *vd = reinterpret_cast<u32x4_t *>(v_cache + dst);
    for (int i = threadIdx.x; i < vecs; i += blockDim.x) {
      kd[i] = ks[i];
      vd[i] = vs[i];
    }
  }
}

// grid.x = pair, grid.y = 0 for K and 1 for V, grid.z = chunk of the block.
// Block dst becomes a copy of block src ("vLLM: Anatomy and Mechanisms",
// section "Memory Sharing via Copy-on-Write (CoW)": only the block where the
// beams diverge is copied).
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint16_t *__restrict__ k_cache,
                                                          uint16_t *__restrict__ v_cache,
                                                          const int64_t *__restrict__ pairs,
                                                          int64_t block_elems, int64_t num_blocks,
                                                          int32_t chunk_vecs) {
  const int64_t src = pairs[2 * (size_t)blockIdx.x];
  const int64_t dst = pairs[2 * (size_t)blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint16_t *cache = blockIdx.y ? v_cache : k_cache;
  const u32x4_t *from = reinterpret_cast<const u32x4_t *>(cache + (size_t)src * block_elems);
  u32x4_t *to = reinterpret_cast<u32x4_t *>(cache + (size_t)dst * block_elems);
  const int64_t vecs = block_elems / 8;
  const int64_t lo = (int64_t)blockIdx.z * chunk_vecs;
  const int64_t hi = lo + chunk_vecs < vecs ? lo + chunk_vecs : vecs;
  for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x) to[i] = from[i];
}

// Moves whole blocks between the device cache and a host cache in pinned
// memory (swapping a preempted request's blocks out to host RAM and back:
// "vLLM: Anatomy and Mechanisms of High-Throughput LLM Inference", section
// "Preemption and Recovery"; "vLLM Internals", section "The Block Manager").
// `from_*` and `to_*` are the two sides (device addresses of the host
// arrays); grid = (pair, K/V, 32 KiB chunk of a block). A pair with an index
// outside its side's pool is skipped. Over PCIe every workgroup keeps its
// chunk's 16-byte loads in flight together.
__global__ __launch_bounds__(256) void swap_blocks_kernel(const uint16_t *__restrict__ from_k,
                                                          const uint16_t *__restrict__ from_v,
                                                          int64_t from_blocks, uint16_t *__restrict__ to_k,
                                                          uint16_t *__restrict__ to_v, int64_t to_blocks,
                                                          const int64_t *__restrict__ pairs, int64_t block_elems,
                                                          int32_t chunk_vecs) {
  const int64_t src = pairs[2 * (size_t)blockIdx.x];
  const int64_t dst = pairs[2 * (size_t)blockIdx.x + 1];
  if (src < 0 || src >= from_blocks || dst < 0 || dst >= to_blocks) return;
  const u32x4_t *from = reinterpret_cast<const u32x4_t *>((blockIdx.y ? from_v : from_k) + (size_t)src * block_elems);
  u32x4_t *to = reinterpret_cast<u32x4_t *>((blockIdx.y ? to_v : to_k) + (size_t)dst * block_elems);
  const int64_t vecs = block_elems / 8;
  const int64_t lo = (int64_t)blockIdx.z * chunk_vecs;
  const int64_t hi = lo + chunk_vecs < vecs ? lo + chunk_vecs : vecs;
  for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x) to[i] = from[i];
}

// Grid-stride 16-byte copy (measurement helper).
__global__ __launch_bounds__(256) void probe_copy_kernel(u32x4_t *__restrict__ dst,
                                                         const u32x4_t *__restrict__ src,
                                                         size_t vecs) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < vecs; i += stride) dst[i] = src[i];
}

// Streaming read folded with xor; one word per thread goes to `sink` so the
// loads cannot be dropped (measurement helper). Wavefronts take 4 KiB chunks
// in grid-stride order and read each as four 1 KiB loads, the first with the
// non-temporal hint, so a quarter of the cache lines stream with the hint
// (the decode kernel's mix; on MI355X it reads 1.26 GB at about 6.4 TB/s,
// against about 5.95 TB/s with plain loads only). A tail short of a chunk
// is read by plain grid-stride loads.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4_t *__restrict__ src,
                                                         size_t vecs, uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t lane = threadIdx.x & 63, wave = tid >> 6, nwaves = stride >> 6;
  const size_t chunks = vecs / 256;  // 256 vectors = 4 KiB
  u32x4_t acc = {0, 0, 0, 0};
  for (size_t c = wave; c < chunks; c += nwaves) {
    const u32x4_t *p = src + c * 256 + lane;
    acc ^= __builtin_nontemporal_load(p);
    acc ^= p[64];
    acc ^= p[128];
    acc ^= p[192];
  }
  for (size_t i = chunks * 256 + tid; i < vecs; i += stride) acc ^= src[i];
  sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

hipError_t launch_reshape_and_cache(const uint16_t *k, const uint16_t *v, const int64_t *slots,
                                    uint16_t *k_cache, uint16_t *v_cache, int32_t num_tokens,
                                    int32_t row_elems, int64_t num_slots, hipStream_t stream) {
  const int vecs = row_elems / 8;
  const int threads = vecs >= 256 ? 256 : ((vecs + 63) / 64) * 64;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)num_tokens), dim3(threads), 0, stream,
                     k, v, slots, k_cache, v_cache, row_elems, num_slots);
  return hipGetLastError();
}

hipError_t launch_step_scatter(const uint16_t *k, const uint16_t *v, const int32_t *tables, const int32_t *lens,
                               uint16_t *k_cache, uint16_t *v_cache, int32_t num_seqs, int32_t row_elems,
                               int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks,
                               hipStream_t stream) {
  if (num_seqs <= 0) return hipSuccess;
  const int32_t threads = row_elems / 8 < 256 ? ((row_elems / 8 + 63) / 64) * 64 : 256;
  const unsigned grid = (unsigned)(num_seqs < 4096 ? num_seqs : 4096);
  hipLaunchKernelGGL(step_scatter_kernel, dim3(grid), dim3(threads), 0, stream, k, v, tables, lens, k_cache,
                     v_cache, num_seqs, row_elems, max_blocks_per_seq, block_size, num_blocks);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(uint16_t *k_cache, uint16_t *v_cache, const int64_t *pairs,
                              int32_t num_pairs, int64_t block_elems, int64_t num_blocks,
                              hipStream_t stream) {
  const int64_t vecs = block_elems / 8;
  const int32_t chunk = 2048;  // 32 KiB of a block per workgroup
  const unsigned chunks = (unsigned)((vecs + chunk - 1) / chunk);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, 2, chunks), dim3(256), 0, stream,
                     k_cache, v_cache, pairs, block_elems, num_blocks, chunk);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const uint16_t *from_k, const uint16_t *from_v, int64_t from_blocks, uint16_t *to_k,
                              uint16_t *to_v, int64_t to_blocks, const int64_t *pairs, int32_t num_pairs,
                              int64_t block_elems, hipStream_t stream) {
  const int64_t vecs = block_elems / 8;
  const int32_t chunk = 2048;  // 32 KiB of a block per workgroup
  const unsigned chunks = (unsigned)((vecs + chunk - 1) / chunk);
  hipLaunchKernelGGL(swap_blocks_kernel, dim3((unsigned)num_pairs, 2, chunks), dim3(256), 0, stream, from_k, from_v,
                     from_blocks, to_k, to_v, to_blocks, pairs, block_elems, chunk);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void *dst, const void *src, size_t bytes, hipStream_t stream) {
  const size_t vecs = bytes / 16;
  size_t blocks = (vecs + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<u32x4_t *>(dst), static_cast<const u32x4_t *>(src), vecs);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
  const size_t vecs = bytes / 16;
  if (vecs == 0) return hipSuccess;
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeReadBlocks), dim3(256), 0, stream,
                     static_cast<const u32x4_t *>(src), vecs, sink);
  return hipGetLastError();
}

}  // namespace pa
