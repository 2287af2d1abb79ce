// C-ABI front end of libpa.so: argument checks, decode planning, workspace
// handling and launches. Every check here runs on the host before any HIP
// call, so argument errors are reported without a GPU.

#include <stdlib.h>
#include <string.h>

#include <string>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const std::string &msg) {
  g_error = msg;
  return code;
}

int ok() {
  g_error.clear();
  return PA_OK;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Workgroups per decode call. The units (blocks x head groups) are shared
// evenly by all workgroups, so the count only sets how much of the chip is
// busy and how many segments get cut. One wavefront per SIMD, 4 per compute
// unit on a 256-CU MI355X: two wavefronts on one SIMD compete for issue,
// and the older one runs ahead while the younger one finishes alone with
// half the loads in flight. So floor(4 / heads_per_wg) workgroups per CU,
// all resident at once (a second round of workgroups would undo the
// balance). Fewer when every sequence at max_blocks_per_seq (as chunks) would still give
// a workgroup fewer than 4 units. The count depends on the sizes only (not on
// the device or the data), so workspace sizes are a host function and
// results are reproducible. PA_DECODE_WGS overrides it (tests, tuning).
// Launches with more than 32 columns per KV head (a workgroup per head group
// of column groups) are heavier on the matrix cores and run two wavefronts
// per SIMD, 8 per compute unit.
constexpr int64_t kTargetCUs = 256;
constexpr int64_t kWavesPerCU = 4;
constexpr int64_t kWideWavesPerCU = 8;
// One-wavefront workgroups (one KV head per head group) on one column tile
// run three per compute unit when the call has at most kFewSegments
// (sequence, head group) segments: long segments are then cut at every
// workgroup boundary, and a fourth wavefront per unit adds pieces, records
// and merge work without adding bandwidth. Measured on one KV head, 4 query
// heads, 32-256 sequences of 1-16K tokens (132-264 MB): the fused step 4-10%
// faster than with four (one GPU's share of the GQA layer at 8-way tensor
// parallelism: 32.9 against 34.2 us), the same at 512 sequences; with 1536
// and more short sequences four per unit stay faster (4096 of median 64
// tokens: 55.8 against 61.7 us).
constexpr int64_t kFewSegmentWavesPerCU = 3;
constexpr int64_t kFewSegments = 512;

int32_t decode_wgs(int64_t num_seqs, int32_t num_head_groups, int32_t heads_per_wg,
                   int32_t max_chunks_per_seq, int64_t waves_per_cu = kWavesPerCU) {
  int64_t w = kTargetCUs * (waves_per_cu / heads_per_wg > 0 ? waves_per_cu / heads_per_wg : 1);
  const int64_t units_bound = num_seqs * num_head_groups * (int64_t)max_chunks_per_seq;
  const int64_t by_work = (units_bound + 3) / 4;
  if (by_work < w) w = by_work;
  if (const char *env = getenv("PA_DECODE_WGS")) {
    const long v = strtol(env, nullptr, 10);
    if (v > 0) w = v;
  }
  if (w < 1) w = 1;
  if (w > (1 << 20)) w = 1 << 20;
  return (int32_t)w;
}

// Which ALU computes a single-token decode with one query head per KV head.
// The matrix-core tiles carry 16 query-head columns, of which one is live
// here; the vector path computes the one column on the vector ALU. Measured
// on the MHA layer (64 sequences, 32/32 heads), the two run in the same time
// (decode kernel 216.1 against 216.3 us; the call is bound by memory), so
// the matrix cores, which do not win, are not used for it.
// PA_DECODE_PATH=mfma|vector overrides the default (tests, tuning).
constexpr bool kVectorPathDefault = true;

int32_t use_vector_path(int32_t group, int32_t q_len) {
  if (group != 1 || q_len != 1) return 0;
  if (const char *env = getenv("PA_DECODE_PATH")) {
    if (!strcmp(env, "vector")) return 1;
    if (!strcmp(env, "mfma")) return 0;
  }
  return kVectorPathDefault ? 1 : 0;
}

// KV heads per workgroup (one wavefront each): the largest divisor of
// num_kv_heads that is <= 4.
int32_t heads_per_workgroup(int32_t num_kv_heads) {
  for (int32_t h = 4; h > 1; --h)
    if (num_kv_heads % h == 0) return h;
  return 1;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The kernels move data in 16-byte vectors.
int check_aligned(const void *p, const char *what) {
  if (reinterpret_cast<uintptr_t>(p) % 16) return fail(PA_ERR_UNSUPPORTED, std::string(what) + " must be 16-byte aligned");
  return PA_OK;
}

int check_cache(const pa_kv_cache *c, bool need_data) {
  if (!c) return fail(PA_ERR_NULL, "cache descriptor is NULL");
  if (need_data && (!c->k_cache || !c->v_cache)) return fail(PA_ERR_NULL, "k_cache or v_cache is NULL");
  if (need_data && (check_aligned(c->k_cache, "k_cache") != PA_OK || check_aligned(c->v_cache, "v_cache") != PA_OK))
    return PA_ERR_UNSUPPORTED;
  if (c->dtype != PA_DTYPE_BF16) return fail(PA_ERR_UNSUPPORTED, "only bf16 caches are supported");
  if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "block_size must be 8, 16 or 32");
  if (c->head_size != 64 && c->head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_size must be 64 or 128");
  if (c->num_blocks < 1) return fail(PA_ERR_SHAPE, "num_blocks must be >= 1");
  if (c->num_kv_heads < 1) return fail(PA_ERR_SHAPE, "num_kv_heads must be >= 1");
  // Kernels address a block with 32-bit byte offsets.
  if ((int64_t)c->num_kv_heads * c->head_size * c->block_size * 2 > (int64_t)1 << 30)
    return fail(PA_ERR_SHAPE, "a cache block (block_size * num_kv_heads * head_size * 2 bytes) exceeds 1 GiB");
  return PA_OK;
}

int check_decode_shape(const pa_kv_cache *c, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_blocks_per_seq) {
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs < 0");
  if (max_blocks_per_seq < 1) return fail(PA_ERR_SHAPE, "max_blocks_per_seq must be >= 1");
  if (num_q_heads < 1 || num_q_heads % c->num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "num_q_heads must be a positive multiple of num_kv_heads");
  if (num_q_heads / c->num_kv_heads > 16)
    return fail(PA_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
  if ((int64_t)max_blocks_per_seq * c->block_size > 0x7fffffffLL)
    return fail(PA_ERR_SHAPE, "max_blocks_per_seq too large");
  if ((int64_t)num_seqs * c->num_kv_heads > 0x7fffffffLL)
    return fail(PA_ERR_SHAPE, "num_seqs * num_kv_heads too large");
  // The kernels read the context lengths through one buffer resource, whose
  // range is a 32-bit byte count.
  if (num_seqs > pa::kMaxDecodeSeqs) return fail(PA_ERR_UNSUPPORTED, "more than 2^28 sequences");
  return PA_OK;
}

// Several new tokens per sequence: their (token, query head) pairs of one KV
// head are the columns of the launch, at most 8 column groups of 32.
int check_q_len(const pa_kv_cache *c, int32_t num_q_heads, int32_t q_len) {
  if (q_len < 1) return fail(PA_ERR_SHAPE, "q_len must be >= 1");
  if ((int64_t)q_len * (num_q_heads / c->num_kv_heads) > pa::kMaxDecodeCols)
    return fail(PA_ERR_UNSUPPORTED, "q_len * (num_q_heads / num_kv_heads) must be <= 256");
  return PA_OK;
}

// The decode kernel works in chunks of 16 tokens: a table row of
// max_blocks_per_seq blocks holds at most this many.
int32_t chunks_per_row(const pa_kv_cache *c, int32_t max_blocks_per_seq) {
  return (int32_t)(((int64_t)max_blocks_per_seq * c->block_size + 15) / 16);
}

// The fused step reads each sequence's newest position as one more chunk.
int32_t step_chunks_per_row(const pa_kv_cache *c, int32_t max_blocks_per_seq, bool fused) {
  return chunks_per_row(c, max_blocks_per_seq) + (fused ? 1 : 0);
}

// Sharing-aware decode: an item serves up to 32 / group sequences (its
// columns are their query heads of one KV head: at most two MFMA tiles).
int32_t members_per_item(int32_t group) { return 32 / group; }

// Workspace of the sharing-aware calls: header, segments (+ sentinel),
// member records (two ints per sequence), merge records (one per
// workgroup), then the partial records of cut segments (2 per workgroup).
struct SharedLayout {
  pa::DecodePlan plan;
  int32_t cols;
  size_t items_off, members_off, desc_off, ml_off, o_off, total;
};

SharedLayout layout_shared(const pa_kv_cache *c, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq) {
  SharedLayout l{};
  const int32_t group = num_q_heads / c->num_kv_heads;
  l.plan.heads_per_wg = heads_per_workgroup(c->num_kv_heads);
  l.plan.num_head_groups = c->num_kv_heads / l.plan.heads_per_wg;
  l.plan.col_groups = 1;
  // A segment holds at most a table row's chunks per member.
  l.plan.num_wgs = decode_wgs(num_seqs, l.plan.num_head_groups, l.plan.heads_per_wg, chunks_per_row(c, max_blocks_per_seq));
  l.cols = members_per_item(group) * group;
  l.plan.rec_cols = l.cols;
  const size_t rows = 2 * (size_t)l.plan.num_wgs * l.plan.heads_per_wg * l.cols;
  l.items_off = 256;  // ShareHeader
  l.members_off = l.items_off + round_up(((size_t)num_seqs + 1) * sizeof(pa::ShareItem), 256);
  l.desc_off = l.members_off + round_up((size_t)num_seqs * 2 * sizeof(int32_t), 256);
  l.ml_off = l.desc_off + round_up((size_t)l.plan.num_wgs * sizeof(int4), 256);
  l.o_off = l.ml_off + round_up(rows * 2 * sizeof(float), 256);
  l.total = l.o_off + round_up(rows * c->head_size * sizeof(float), 256);
  return l;
}

int check_shared(const pa_kv_cache *c, int32_t num_seqs, int32_t num_groups) {
  if (num_seqs > pa::kMaxSharedSeqs)
    return fail(PA_ERR_UNSUPPORTED, "sharing-aware decode takes at most 4096 sequences");
  if (num_groups < 0 || num_groups > num_seqs) return fail(PA_ERR_SHAPE, "num_groups must be in 0..num_seqs");
  return PA_OK;
}

// The checks every sharing-aware call makes on its shape.
int check_shared_shape(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                       int32_t num_groups, bool data) {
  int rc = check_cache(cache, data);
  if (rc != PA_OK) return rc;
  rc = check_decode_shape(cache, num_seqs, num_q_heads, max_blocks_per_seq);
  if (rc != PA_OK) return rc;
  return check_shared(cache, num_seqs, num_groups);
}

// Launches the plan kernel into a plan buffer laid out as the front of a
// SharedLayout (header, segments, member records).
hipError_t launch_plan(const pa_kv_cache *cache, const SharedLayout &l, const int32_t *context_lens, int32_t num_seqs,
                       int32_t num_q_heads, int32_t max_blocks_per_seq, const int32_t *group_starts,
                       const int32_t *shared_blocks, int32_t num_groups, const int32_t *shared_prev, char *plan,
                       hipStream_t hs) {
  pa::SharePlanArgs p{};
  p.lens = context_lens;
  p.group_starts = group_starts;
  p.shared_blocks = shared_blocks;
  p.shared_prev = shared_prev;
  p.members = reinterpret_cast<int32_t *>(plan + l.members_off);
  p.items = reinterpret_cast<pa::ShareItem *>(plan + l.items_off);
  p.share = reinterpret_cast<pa::ShareHeader *>(plan);
  p.num_seqs = num_seqs;
  p.num_groups = shared_prev ? 0 : num_groups;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.group = num_q_heads / cache->num_kv_heads;
  p.members_per_item = members_per_item(p.group);
  p.num_head_groups = l.plan.num_head_groups;
  p.block_size = cache->block_size;
  return pa::launch_share_plan(p, hs);
}

// Launches decode and merge on a plan; `run` is the call's scratch (merge
// records, then partial records), laid out as the back of a SharedLayout.
hipError_t launch_planned(const pa_kv_cache *cache, const SharedLayout &l, const void *q, const int32_t *block_tables,
                          int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq, const char *plan,
                          float scale, void *out, char *run, hipStream_t hs) {
  pa::DecodeArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k_cache = static_cast<const uint16_t *>(cache->k_cache);
  a.v_cache = static_cast<const uint16_t *>(cache->v_cache);
  a.block_tables = block_tables;
  a.context_lens = reinterpret_cast<const int32_t *>(plan + l.members_off);  // the member records
  a.out = static_cast<uint16_t *>(out);
  a.merge_desc = reinterpret_cast<int4 *>(run);
  a.part_ml = reinterpret_cast<float *>(run + (l.ml_off - l.desc_off));
  a.part_o = reinterpret_cast<float *>(run + (l.o_off - l.desc_off));
  a.num_blocks = cache->num_blocks;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = num_q_heads / cache->num_kv_heads;
  a.q_len = 1;
  a.num_cols = l.cols;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = cache->block_size;
  a.heads_per_wg = l.plan.heads_per_wg;
  a.num_head_groups = l.plan.num_head_groups;
  a.col_groups = 1;
  a.rec_cols = l.cols;
  a.num_wgs = l.plan.num_wgs;
  a.scale_log2 = scale * 1.44269504088896340736f;
  a.items = reinterpret_cast<const pa::ShareItem *>(plan + l.items_off);
  a.share = reinterpret_cast<const pa::ShareHeader *>(plan);
  return pa::launch_decode_planned(a, cache->head_size, hs);
}

// Checks, plans and launches a sharing-aware call: the group form, or
// (shared_prev non-null) the chain form. The workspace holds the plan, then
// the call's scratch.
int shared_impl(const pa_kv_cache *cache, const void *q, const int32_t *block_tables, const int32_t *context_lens,
                int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq, const int32_t *group_starts,
                const int32_t *shared_blocks, int32_t num_groups, const int32_t *shared_prev, float scale, void *out,
                void *workspace, size_t workspace_bytes, void *stream) {
  const char *name = shared_prev ? "pa_decode_shared_tree" : "pa_decode_shared";
  int rc = check_shared_shape(cache, num_seqs, num_q_heads, max_blocks_per_seq, num_groups, num_seqs > 0);
  if (rc != PA_OK) return rc;
  if (num_seqs == 0) return ok();
  if (!q || !block_tables || !context_lens || !out)
    return fail(PA_ERR_NULL, "q, block_tables, context_lens or out is NULL");
  if (check_aligned(q, "q") != PA_OK || check_aligned(out, "out") != PA_OK) return PA_ERR_UNSUPPORTED;
  if (num_groups > 0 && !shared_prev && (!group_starts || !shared_blocks))
    return fail(PA_ERR_NULL, "group_starts or shared_blocks is NULL");

  const SharedLayout l = layout_shared(cache, num_seqs, num_q_heads, max_blocks_per_seq);
  if (workspace && workspace_bytes < l.total)
    return fail(PA_ERR_WORKSPACE, std::string("workspace smaller than ") + name + "_workspace_bytes()");
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(PA_ERR_WORKSPACE, "workspace must be 16-byte aligned");

  hipStream_t hs = static_cast<hipStream_t>(stream);
  void *ws = workspace;
  bool owned = false;
  if (!ws) {
    hipError_t e = hipMallocAsync(&ws, l.total, hs);
    if (e != hipSuccess) return hip_fail(e, "hipMallocAsync(workspace)");
    owned = true;
  }
  char *base = static_cast<char *>(ws);
  hipError_t e = launch_plan(cache, l, context_lens, num_seqs, num_q_heads, max_blocks_per_seq, group_starts,
                             shared_blocks, num_groups, shared_prev, base, hs);
  if (e == hipSuccess)
    e = launch_planned(cache, l, q, block_tables, num_seqs, num_q_heads, max_blocks_per_seq, base, scale, out,
                       base + l.desc_off, hs);
  if (owned) {
    hipError_t fe = hipFreeAsync(ws, hs);
    if (e == hipSuccess) e = fe;
  }
  if (e != hipSuccess) return hip_fail(e, (std::string(name) + " launch").c_str());
  return ok();
}

}  // namespace

namespace pa {

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_size, int32_t max_chunks_per_seq, int32_t q_len) {
  DecodePlan p{};
  const int32_t cols = q_len * (num_q_heads / num_kv_heads);
  if (cols > pa::kMaxNarrowCols) {
    // One workgroup per KV head of a piece, one wavefront per 32 columns.
    p.col_groups = (cols + 31) / 32;
    p.rec_cols = 32;
    p.heads_per_wg = p.col_groups;
    p.num_head_groups = num_kv_heads;
    p.num_wgs = decode_wgs(num_seqs, p.num_head_groups, p.heads_per_wg, max_chunks_per_seq, kWideWavesPerCU);
  } else {
    p.col_groups = 1;
    p.rec_cols = cols;
    p.heads_per_wg = heads_per_workgroup(num_kv_heads);
    p.num_head_groups = num_kv_heads / p.heads_per_wg;
    const bool few = p.heads_per_wg == 1 && cols <= 16 && (int64_t)num_seqs * p.num_head_groups <= kFewSegments;
    p.num_wgs = decode_wgs(num_seqs, p.num_head_groups, p.heads_per_wg, max_chunks_per_seq,
                           few ? kFewSegmentWavesPerCU : kWavesPerCU);
  }
  if (p.num_wgs <= 1) return p;
  const size_t rows = (size_t)p.num_wgs * 2 * p.heads_per_wg * p.rec_cols;
  p.desc_bytes = round_up((size_t)p.num_wgs * sizeof(int4), 256);
  p.ml_bytes = round_up(rows * 2 * sizeof(float), 256);
  p.o_bytes = round_up(rows * head_size * sizeof(float), 256);
  p.total_bytes = p.desc_bytes + p.ml_bytes + p.o_bytes;
  return p;
}

}  // namespace pa

namespace {

// Checks, plans and launches a decode call. The partial records go to the
// caller's workspace, to stream-ordered scratch allocated here when that is
// NULL, or (static_scratch) to the library's static device scratch, with no
// allocation at all.
int decode_impl(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                const int32_t *context_lens, int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                int32_t max_blocks_per_seq, float scale, void *out, void *workspace,
                size_t workspace_bytes, void *stream, bool static_scratch, const void *k_new = nullptr,
                const void *v_new = nullptr) {
  int rc = check_cache(cache, num_seqs > 0);
  if (rc != PA_OK) return rc;
  rc = check_decode_shape(cache, num_seqs, num_q_heads, max_blocks_per_seq);
  if (rc != PA_OK) return rc;
  rc = check_q_len(cache, num_q_heads, q_len);
  if (rc != PA_OK) return rc;
  if (num_seqs == 0) return ok();
  if (!q || !block_tables || !context_lens || !out)
    return fail(PA_ERR_NULL, "q, block_tables, context_lens or out is NULL");
  if (check_aligned(q, "q") != PA_OK || check_aligned(out, "out") != PA_OK) return PA_ERR_UNSUPPORTED;
  const bool fused = k_new || v_new;
  if (fused && (!k_new || !v_new)) return fail(PA_ERR_NULL, "k or v is NULL");
  if (fused && (check_aligned(k_new, "k") != PA_OK || check_aligned(v_new, "v") != PA_OK)) return PA_ERR_UNSUPPORTED;

  const pa::DecodePlan plan = pa::plan_decode(num_seqs, num_q_heads, cache->num_kv_heads, cache->head_size,
                                              step_chunks_per_row(cache, max_blocks_per_seq, fused), q_len);
  // The decode step in one launch stages each finished sequence's output and
  // new K/V row in LDS until its stream ends. With more sequences per
  // workgroup than it has places for, the rest are stored mid-stream, which
  // delays the waits for the loads around them. Then the new rows go to
  // their slots in a scatter launch first, and the decode launch (still
  // attending over each new token from k and v) stages outputs only, in the
  // room the new rows took. Both forms give the same output and cache.
  const int32_t places = fused ? pa::decode_stage_slots(num_q_heads / cache->num_kv_heads, cache->head_size,
                                                         cache->block_size, true)
                               : 0;
  const bool split_step = fused && places > 0 &&
                          (int64_t)num_seqs * plan.num_head_groups > (int64_t)plan.num_wgs * places;
  if (workspace && workspace_bytes < plan.total_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace smaller than pa_decode_workspace_bytes()");
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(PA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  if (static_scratch && plan.total_bytes > pa::kNoAllocScratchBytes)
    return fail(PA_ERR_WORKSPACE, "this call needs " + std::to_string(plan.total_bytes) +
                                      " bytes of scratch, more than the library's static " +
                                      std::to_string(pa::kNoAllocScratchBytes) + "-byte scratch");

  hipStream_t hs = static_cast<hipStream_t>(stream);
  void *ws = workspace;
  bool owned = false;
  if (static_scratch) {
    if (plan.total_bytes) {
      hipError_t e = pa::noalloc_scratch(&ws);
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    }
  } else if (plan.total_bytes && !ws) {
    hipError_t e = hipMallocAsync(&ws, plan.total_bytes, hs);
    if (e != hipSuccess) return hip_fail(e, "hipMallocAsync(workspace)");
    owned = true;
  }

  pa::DecodeArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k_cache = static_cast<const uint16_t *>(cache->k_cache);
  a.v_cache = static_cast<const uint16_t *>(cache->v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = static_cast<uint16_t *>(out);
  if (plan.total_bytes) {
    char *base = static_cast<char *>(ws);
    a.merge_desc = reinterpret_cast<int4 *>(base);
    a.part_ml = reinterpret_cast<float *>(base + plan.desc_bytes);
    a.part_o = reinterpret_cast<float *>(base + plan.desc_bytes + plan.ml_bytes);
  }
  a.k_new = static_cast<const uint16_t *>(k_new);
  a.v_new = static_cast<const uint16_t *>(v_new);
  a.write_new = split_step ? 0 : 1;
  a.num_blocks = cache->num_blocks;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = num_q_heads / cache->num_kv_heads;
  a.q_len = q_len;
  a.num_cols = q_len * a.group;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = cache->block_size;
  a.heads_per_wg = plan.heads_per_wg;
  a.num_head_groups = plan.num_head_groups;
  a.col_groups = plan.col_groups;
  a.rec_cols = plan.rec_cols;
  a.num_wgs = plan.num_wgs;
  a.scale_log2 = scale * 1.44269504088896340736f;
  a.vector_path = use_vector_path(a.group, q_len);

  hipError_t e = hipSuccess;
  if (split_step)
    e = pa::launch_step_scatter(static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new),
                                block_tables, context_lens, static_cast<uint16_t *>(cache->k_cache),
                                static_cast<uint16_t *>(cache->v_cache), num_seqs,
                                cache->num_kv_heads * cache->head_size, max_blocks_per_seq, cache->block_size,
                                cache->num_blocks, hs);
  if (e == hipSuccess) e = pa::launch_decode(a, cache->head_size, hs);
  if (owned) {
    hipError_t fe = hipFreeAsync(ws, hs);
    if (e == hipSuccess) e = fe;
  }
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

}  // namespace

extern "C" {

const char *pa_last_error(void) { return g_error.c_str(); }

size_t pa_decode_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_blocks_per_seq) {
  return pa_decode_multi_workspace_bytes(cache, num_seqs, 1, num_q_heads, max_blocks_per_seq);
}

size_t pa_decode_multi_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t q_len,
                                       int32_t num_q_heads, int32_t max_blocks_per_seq) {
  if (check_cache(cache, false) != PA_OK) return 0;
  if (check_decode_shape(cache, num_seqs, num_q_heads, max_blocks_per_seq) != PA_OK) return 0;
  if (check_q_len(cache, num_q_heads, q_len) != PA_OK) return 0;
  return pa::plan_decode(num_seqs, num_q_heads, cache->num_kv_heads, cache->head_size,
                         chunks_per_row(cache, max_blocks_per_seq), q_len)
      .total_bytes;
}

int pa_decode(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
              const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
              int32_t max_blocks_per_seq, float scale, void *out, void *workspace,
              size_t workspace_bytes, void *stream) {
  return pa_decode_multi(cache, q, block_tables, context_lens, num_seqs, 1, num_q_heads, max_blocks_per_seq,
                         scale, out, workspace, workspace_bytes, stream);
}

int pa_decode_multi(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                    const int32_t *context_lens, int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                    int32_t max_blocks_per_seq, float scale, void *out, void *workspace,
                    size_t workspace_bytes, void *stream) {
  return decode_impl(cache, q, block_tables, context_lens, num_seqs, q_len, num_q_heads, max_blocks_per_seq, scale,
                     out, workspace, workspace_bytes, stream, false);
}

int pa_decode_step(const pa_kv_cache *cache, const void *q, const void *k, const void *v,
                   const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                   int32_t max_blocks_per_seq, float scale, void *out, void *workspace, size_t workspace_bytes,
                   void *stream) {
  if (num_seqs > 0 && (!k || !v)) return fail(PA_ERR_NULL, "k or v is NULL");
  return decode_impl(cache, q, block_tables, context_lens, num_seqs, 1, num_q_heads, max_blocks_per_seq, scale, out,
                     workspace, workspace_bytes, stream, false, num_seqs > 0 ? k : nullptr,
                     num_seqs > 0 ? v : nullptr);
}

size_t pa_decode_step_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t max_blocks_per_seq) {
  if (check_cache(cache, false) != PA_OK) return 0;
  if (check_decode_shape(cache, num_seqs, num_q_heads, max_blocks_per_seq) != PA_OK) return 0;
  return pa::plan_decode(num_seqs, num_q_heads, cache->num_kv_heads, cache->head_size,
                         step_chunks_per_row(cache, max_blocks_per_seq, true), 1)
      .total_bytes;
}

int pa_decode_noalloc(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                      const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_blocks_per_seq, float scale, void *out, void *stream) {
  return decode_impl(cache, q, block_tables, context_lens, num_seqs, 1, num_q_heads, max_blocks_per_seq, scale,
                     out, nullptr, 0, stream, true);
}

size_t pa_decode_shared_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t max_blocks_per_seq, int32_t num_groups) {
  if (check_cache(cache, false) != PA_OK) return 0;
  if (check_decode_shape(cache, num_seqs, num_q_heads, max_blocks_per_seq) != PA_OK) return 0;
  if (check_shared(cache, num_seqs, num_groups) != PA_OK || num_seqs == 0) return 0;
  return layout_shared(cache, num_seqs, num_q_heads, max_blocks_per_seq).total;
}

int pa_decode_shared(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                     const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_blocks_per_seq, const int32_t *group_starts, const int32_t *shared_blocks,
                     int32_t num_groups, float scale, void *out, void *workspace, size_t workspace_bytes,
                     void *stream) {
  return shared_impl(cache, q, block_tables, context_lens, num_seqs, num_q_heads, max_blocks_per_seq, group_starts,
                     shared_blocks, num_groups, nullptr, scale, out, workspace, workspace_bytes, stream);
}

size_t pa_decode_shared_tree_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                                             int32_t max_blocks_per_seq) {
  return pa_decode_shared_workspace_bytes(cache, num_seqs, num_q_heads, max_blocks_per_seq, 0);
}

int pa_decode_shared_tree(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                          const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                          int32_t max_blocks_per_seq, const int32_t *shared_prev, float scale, void *out,
                          void *workspace, size_t workspace_bytes, void *stream) {
  if (num_seqs > 0 && !shared_prev) return fail(PA_ERR_NULL, "shared_prev is NULL");
  return shared_impl(cache, q, block_tables, context_lens, num_seqs, num_q_heads, max_blocks_per_seq, nullptr,
                     nullptr, 0, shared_prev, scale, out, workspace, workspace_bytes, stream);
}

size_t pa_share_plan_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                           int32_t max_blocks_per_seq) {
  if (check_shared_shape(cache, num_seqs, num_q_heads, max_blocks_per_seq, 0, false) != PA_OK || num_seqs == 0)
    return 0;
  return layout_shared(cache, num_seqs, num_q_heads, max_blocks_per_seq).desc_off;
}

int pa_share_plan(const pa_kv_cache *cache, const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                  int32_t max_blocks_per_seq, const int32_t *group_starts, const int32_t *shared_blocks,
                  int32_t num_groups, const int32_t *shared_prev, void *plan, size_t plan_bytes, void *stream) {
  int rc = check_shared_shape(cache, num_seqs, num_q_heads, max_blocks_per_seq, shared_prev ? 0 : num_groups, false);
  if (rc != PA_OK) return rc;
  if (num_seqs == 0) return ok();
  if (!context_lens || !plan) return fail(PA_ERR_NULL, "context_lens or plan is NULL");
  if (!shared_prev && num_groups > 0 && (!group_starts || !shared_blocks))
    return fail(PA_ERR_NULL, "group_starts or shared_blocks is NULL");
  const SharedLayout l = layout_shared(cache, num_seqs, num_q_heads, max_blocks_per_seq);
  if (plan_bytes < l.desc_off) return fail(PA_ERR_WORKSPACE, "plan smaller than pa_share_plan_bytes()");
  if (reinterpret_cast<uintptr_t>(plan) % 16) return fail(PA_ERR_WORKSPACE, "plan must be 16-byte aligned");
  const hipError_t e = launch_plan(cache, l, context_lens, num_seqs, num_q_heads, max_blocks_per_seq, group_starts,
                                   shared_blocks, num_groups, shared_prev, static_cast<char *>(plan),
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_share_plan launch");
  return ok();
}

size_t pa_decode_shared_planned_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                                                int32_t max_blocks_per_seq) {
  if (check_shared_shape(cache, num_seqs, num_q_heads, max_blocks_per_seq, 0, false) != PA_OK || num_seqs == 0)
    return 0;
  const SharedLayout l = layout_shared(cache, num_seqs, num_q_heads, max_blocks_per_seq);
  return l.total - l.desc_off;
}

int pa_decode_shared_planned(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                             int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq, const void *plan,
                             float scale, void *out, void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_shared_shape(cache, num_seqs, num_q_heads, max_blocks_per_seq, 0, num_seqs > 0);
  if (rc != PA_OK) return rc;
  if (num_seqs == 0) return ok();
  if (!q || !block_tables || !plan || !out) return fail(PA_ERR_NULL, "q, block_tables, plan or out is NULL");
  if (check_aligned(q, "q") != PA_OK || check_aligned(out, "out") != PA_OK) return PA_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(plan) % 16) return fail(PA_ERR_WORKSPACE, "plan must be 16-byte aligned");
  const SharedLayout l = layout_shared(cache, num_seqs, num_q_heads, max_blocks_per_seq);
  const size_t need = l.total - l.desc_off;
  if (workspace && workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "workspace smaller than pa_decode_shared_planned_workspace_bytes()");
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(PA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void *ws = workspace;
  bool owned = false;
  if (!ws) {
    hipError_t e = hipMallocAsync(&ws, need, hs);
    if (e != hipSuccess) return hip_fail(e, "hipMallocAsync(workspace)");
    owned = true;
  }
  hipError_t e = launch_planned(cache, l, q, block_tables, num_seqs, num_q_heads, max_blocks_per_seq,
                                static_cast<const char *>(plan), scale, out, static_cast<char *>(ws), hs);
  if (owned) {
    hipError_t fe = hipFreeAsync(ws, hs);
    if (e == hipSuccess) e = fe;
  }
  if (e != hipSuccess) return hip_fail(e, "pa_decode_shared_planned launch");
  return ok();
}

int pa_reshape_and_cache(const pa_kv_cache *cache, const void *k, const void *v,
                         const int64_t *slot_mapping, int32_t num_tokens, void *stream) {
  int rc = check_cache(cache, num_tokens > 0);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens < 0");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping) return fail(PA_ERR_NULL, "k, v or slot_mapping is NULL");
  if (check_aligned(k, "k") != PA_OK || check_aligned(v, "v") != PA_OK) return PA_ERR_UNSUPPORTED;
  const int64_t row = (int64_t)cache->num_kv_heads * cache->head_size;
  if (row > 0x7fffffffLL) return fail(PA_ERR_SHAPE, "num_kv_heads * head_size too large");
  hipError_t e = pa::launch_reshape_and_cache(
      static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), slot_mapping,
      static_cast<uint16_t *>(cache->k_cache), static_cast<uint16_t *>(cache->v_cache), num_tokens,
      (int32_t)row, cache->num_blocks * cache->block_size, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "reshape_and_cache launch");
  return ok();
}

int pa_copy_blocks(const pa_kv_cache *cache, const int64_t *src_dst_pairs, int32_t num_pairs,
                   void *stream) {
  int rc = check_cache(cache, num_pairs > 0);
  if (rc != PA_OK) return rc;
  if (num_pairs < 0) return fail(PA_ERR_SHAPE, "num_pairs < 0");
  if (num_pairs == 0) return ok();
  if (!src_dst_pairs) return fail(PA_ERR_NULL, "src_dst_pairs is NULL");
  const int64_t block_elems = (int64_t)cache->block_size * cache->num_kv_heads * cache->head_size;
  hipError_t e = pa::launch_copy_blocks(static_cast<uint16_t *>(cache->k_cache),
                                        static_cast<uint16_t *>(cache->v_cache), src_dst_pairs,
                                        num_pairs, block_elems, cache->num_blocks,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
  return ok();
}

// The device address of a host array, if the HIP runtime knows it as pinned
// host memory that kernels may access; nullptr otherwise (so a pageable
// pointer is an error here, never a fault in the kernel).
static void *pinned_device_address(void *host) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, host) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost) return nullptr;
  void *dev = nullptr;
  if (hipHostGetDevicePointer(&dev, host, 0) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return dev;
}

int pa_swap_blocks(const pa_kv_cache *cache, void *host_k, void *host_v, int64_t host_num_blocks,
                   const int64_t *src_dst_pairs, int32_t num_pairs, int32_t direction, void *stream) {
  int rc = check_cache(cache, num_pairs > 0);
  if (rc != PA_OK) return rc;
  if (num_pairs < 0) return fail(PA_ERR_SHAPE, "num_pairs < 0");
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_ERR_SHAPE, "direction must be PA_SWAP_OUT or PA_SWAP_IN");
  if (host_num_blocks < 0) return fail(PA_ERR_SHAPE, "host_num_blocks < 0");
  if (num_pairs == 0) return ok();
  if (!host_k || !host_v || !src_dst_pairs) return fail(PA_ERR_NULL, "host_k, host_v or src_dst_pairs is NULL");
  uint16_t *hk = static_cast<uint16_t *>(pinned_device_address(host_k));
  uint16_t *hv = static_cast<uint16_t *>(pinned_device_address(host_v));
  if (!hk || !hv)
    return fail(PA_ERR_UNSUPPORTED, "host_k and host_v must be pinned host memory (hipHostMalloc)");
  const int64_t block_elems = (int64_t)cache->block_size * cache->num_kv_heads * cache->head_size;
  uint16_t *dk = static_cast<uint16_t *>(cache->k_cache);
  uint16_t *dv = static_cast<uint16_t *>(cache->v_cache);
  hipError_t e = direction == PA_SWAP_OUT
                     ? pa::launch_swap_blocks(dk, dv, cache->num_blocks, hk, hv, host_num_blocks, src_dst_pairs,
                                              num_pairs, block_elems, static_cast<hipStream_t>(stream))
                     : pa::launch_swap_blocks(hk, hv, host_num_blocks, dk, dv, cache->num_blocks, src_dst_pairs,
                                              num_pairs, block_elems, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "swap_blocks launch");
  return ok();
}

int pa_probe_copy(void *dst, const void *src, size_t bytes, void *stream) {
  if (bytes == 0) return ok();
  if (!dst || !src) return fail(PA_ERR_NULL, "dst or src is NULL");
  if (bytes % 16 || (reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) % 16)
    return fail(PA_ERR_SHAPE, "probe copy needs 16-byte sizes and alignment");
  hipError_t e = pa::launch_probe_copy(dst, src, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "probe copy launch");
  return ok();
}

size_t pa_probe_read_sink_bytes(void) { return (size_t)pa::kProbeReadBlocks * 256 * sizeof(uint32_t); }

int pa_probe_read(const void *src, size_t bytes, void *sink, size_t sink_bytes, void *stream) {
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(PA_ERR_NULL, "src or sink is NULL");
  if (bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return fail(PA_ERR_SHAPE, "probe read needs 16-byte sizes and alignment");
  if (sink_bytes < pa_probe_read_sink_bytes())
    return fail(PA_ERR_WORKSPACE, "sink smaller than pa_probe_read_sink_bytes()");
  hipError_t e = pa::launch_probe_read(src, bytes, static_cast<uint32_t *>(sink),
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "probe read launch");
  return ok();
}

}  // extern "C"
