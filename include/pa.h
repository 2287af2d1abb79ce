/*
 * pa.h - C ABI of the MI355X (gfx950) paged KV-cache decode library (libpa.so).
 *
 * The library implements the data-parallel hot path of a decode step over a
 * KV cache kept in fixed-size, non-contiguous physical blocks:
 *
 *   - "vLLM: Anatomy and Mechanisms of High-Throughput LLM Inference",
 *     section "PagedAttention: The vLLM Innovation" / "Block-Level
 *     Management": a request's KV cache is split into logical blocks that a
 *     block table maps to physical blocks; 16 tokens per block by default.
 *   - the same page, section "Memory Sharing via Copy-on-Write (CoW)":
 *     sequences share physical blocks and only the block where they diverge
 *     is copied.
 *   - "Inside vLLM: Anatomy of a High-Throughput LLM Inference System",
 *     section "Scheduler": a decode step is a forward pass over the most
 *     recent token, with every earlier K/V vector already cached; section
 *     "LLM Engine constructor": the cache is allocated, reshaped and bound
 *     to the attention layers (here: a caller-owned pa_kv_cache descriptor).
 *
 * Conventions shared by every call:
 *   - Every data pointer is a DEVICE pointer owned by the caller. The library
 *     never frees caller memory and keeps no state between calls, except a
 *     thread-local error string (pa_last_error), per-device launch settings,
 *     and the static scratch of pa_decode_noalloc.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream). A return of PA_OK means the work was enqueued.
 *   - bfloat16 tensors are passed as raw 16-bit storage.
 *   - Errors that can be seen on the host are reported before anything is
 *     enqueued: a NULL pointer, a negative count, an unsupported dtype, head
 *     size, block size or head grouping, a data pointer that is not 16-byte
 *     aligned (the kernels move data in 16-byte vectors), or a workspace that
 *     is too small.
 *     PA_ERR_HIP reports a failed HIP call; its text is in pa_last_error().
 *   - Device-side indices are clamped or skipped, never trusted: a block id
 *     outside [0, num_blocks), a slot outside the pool or a CoW pair outside
 *     the pool never causes an out-of-bounds access. Such input makes the
 *     affected output unspecified; the kernels still finish normally.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* a count or size is negative or inconsistent */
  PA_ERR_UNSUPPORTED = -3, /* dtype, block size, head size or grouping not built */
  PA_ERR_WORKSPACE = -4,   /* workspace given but smaller than required */
  PA_ERR_HIP = -5          /* a HIP runtime call failed */
} pa_status;

enum { PA_DTYPE_BF16 = 0 };

/*
 * The KV cache bound to one attention layer ("Inside vLLM", section "LLM
 * Engine constructor": allocate, reshape and bind). K and V are separate
 * contiguous arrays of shape [num_blocks, block_size, num_kv_heads,
 * head_size]: element (b, t, h, d) is at ((b*block_size + t)*num_kv_heads +
 * h)*head_size + d. One block of one array holds block_size tokens of every
 * KV head, so a block's K plus V is 2*block_size*num_kv_heads*head_size*2
 * bytes, the per-block size the page gives.
 *
 * Supported: dtype PA_DTYPE_BF16; block_size 8, 16 or 32 (every call);
 * head_size 64 or 128;
 * num_blocks >= 1; num_kv_heads >= 1; one block of one array at most 1 GiB;
 * k_cache and v_cache 16-byte aligned. The descriptor is read on every call
 * and not kept.
 */
typedef struct pa_kv_cache {
  void *k_cache;
  void *v_cache;
  int64_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_size;
  int32_t dtype;
} pa_kv_cache;

/*
 * pa_decode - attention of one new query token per sequence over that
 * sequence's paged K/V ("Inside vLLM", section "Scheduler"; block-table
 * indexing from "vLLM: Anatomy and Mechanisms", section "Block-Level
 * Management").
 *
 * For sequence s with n = context_lens[s] cached tokens (the newest one
 * included, so pa_reshape_and_cache of this step runs first), logical token
 * i lives in physical block block_tables[s*max_blocks_per_seq + i/B] at
 * offset i%B, B = cache->block_size. Query head h uses KV head
 * h / (num_q_heads/num_kv_heads).
 *   out[s,h,:] = sum_i softmax_i(scale * q[s,h,:].k_i) * v_i
 * computed with fp32 accumulation and stored as bfloat16 (round to nearest
 * even). n == 0 gives a zero row.
 *
 *   q             bf16 [num_seqs, num_q_heads, head_size], contiguous,
 *                 16-byte aligned
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]; entries at index
 *                 >= ceil(n/B) are never read
 *   context_lens  int32 [num_seqs]; 0 <= n <= max_blocks_per_seq*B
 *                 (larger values are treated as max_blocks_per_seq*B)
 *   num_q_heads   multiple of num_kv_heads, with at most 16 query heads per
 *                 KV head
 *   out           bf16 [num_seqs, num_q_heads, head_size], 16-byte aligned;
 *                 must not alias any input
 *   workspace     device scratch of at least pa_decode_workspace_bytes(...)
 *                 bytes, 16-byte aligned, or NULL. The call shares the K/V
 *                 blocks of the whole batch evenly among its workgroups, so a
 *                 sequence can be cut into pieces; each piece leaves partial
 *                 results (running max, sum, unnormalised output) that a
 *                 second kernel merges with log-sum-exp weights. The
 *                 workspace holds those partials and one merge record per
 *                 workgroup. It needs no
 *                 initialisation: every call rewrites what it reads. Calls
 *                 that share a workspace must not overlap in time (keep them
 *                 on one stream, or order them). With NULL the library
 *                 allocates scratch stream-ordered (hipMallocAsync) and frees
 *                 it after the launch.
 *
 * The output does not depend on where blocks sit in the pool. It is
 * reproducible bit for bit for the same sizes and context lengths (no
 * atomics; the cut points depend only on those).
 *
 * K and V rows at positions < n must be finite: the kernels multiply every
 * value by weights some of which are zero, and an infinity times zero is
 * NaN, which would spread to other head dims. Rows past a context length
 * (stale tail slots) may hold anything, NaN included; they are never read
 * into the sums. With one query head per KV head the arithmetic runs on the
 * vector ALU, otherwise on matrix cores (PA_DECODE_PATH=mfma|vector in the
 * environment overrides the first choice, for tests and tuning).
 *
 * Errors: PA_ERR_NULL (cache, cache->k_cache/v_cache, q, block_tables,
 * context_lens or out NULL while num_seqs > 0), PA_ERR_SHAPE (negative
 * counts, max_blocks_per_seq < 1, num_q_heads % num_kv_heads != 0),
 * PA_ERR_UNSUPPORTED (see pa_kv_cache; group size > 16; q or out not
 * 16-byte aligned; num_seqs > 2^28), PA_ERR_WORKSPACE
 * (too small or misaligned), PA_ERR_HIP. num_seqs == 0 is a no-op.
 */
int pa_decode(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
              const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
              int32_t max_blocks_per_seq, float scale, void *out, void *workspace,
              size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace pa_decode needs for these sizes (0 when the call runs
 * as a single workgroup and nothing is cut). Host-only; depends on the sizes
 * alone, not on the device or the data; returns 0 for invalid sizes.
 */
size_t pa_decode_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_blocks_per_seq);

/*
 * pa_decode_step - one decode step in one call: pa_reshape_and_cache of
 * each sequence's new token, then pa_decode, with the same result
 * ("Inside vLLM", section "Scheduler": a decode step attends from the most
 * recent token over every cached K/V vector, its own included, and stores
 * its K/V for later steps; "vLLM: Anatomy and Mechanisms", section
 * "Block-Level Management": the token's slot lies in the block its table
 * names).
 *
 * Sequence s has one new token, at position n - 1 (n = context_lens[s], the
 * new token included). Its K and V are k[s] and v[s]; its slot is row
 * (n - 1) % B of physical block block_tables[s*max_blocks_per_seq +
 * (n - 1)/B], B = cache->block_size (the slot pa_reshape_and_cache would be
 * given). The call attends over positions 0 .. n - 2 from the cache and
 * over position n - 1 from k[s], v[s], and writes k[s], v[s] into that
 * slot. The output is pa_decode's after that scatter, and the cache after
 * the call is the cache after it, bit for bit. n == 0: nothing is written
 * and the output row is zero. Usually one launch does both; with more
 * sequences per workgroup than that launch can keep in LDS until its stream
 * ends (thousands of short sequences), the new rows are scattered by a
 * launch of their own first, which is faster there. The output and the
 * cache are the same bit for bit either way. A table entry for position n - 1 outside
 * [0, num_blocks) skips the write (the output still uses k[s], v[s]).
 *
 *   k, v   bf16 [num_seqs, num_kv_heads, head_size], 16-byte aligned
 * Other arguments, the workspace (pa_decode_step_workspace_bytes) and the
 * errors are those of pa_decode. Preconditions: the slot's block is not read
 * at that row by another sequence of the call (a copy-on-write block is
 * private before a token is appended to it), and no two sequences share a
 * slot.
 */
int pa_decode_step(const pa_kv_cache *cache, const void *q, const void *k, const void *v,
                   const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                   int32_t num_q_heads, int32_t max_blocks_per_seq, float scale, void *out,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of pa_decode_step (as pa_decode_workspace_bytes). */
size_t pa_decode_step_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_blocks_per_seq);

/*
 * pa_decode_noalloc - pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same arguments, computation, kernels and result (bit
 * for bit) as pa_decode, without the workspace arguments: the partial
 * results go to a static device array of the library (PA_NOALLOC_SCRATCH_BYTES,
 * 16.5 MiB), which each GPU the library runs on holds until the process
 * ends. The call allocates nothing: no hipMalloc, no hipMallocAsync, no
 * free. The caller still owns q, block_tables, context_lens and out.
 *
 * The scratch is one array per GPU, shared by every call on that GPU: two
 * calls on one GPU that overlap in time (different streams, unordered) race
 * on it and their results are undefined. Order them (one stream, or events).
 * It needs no initialisation: every call rewrites what it reads.
 *
 * Errors: those of pa_decode, and PA_ERR_WORKSPACE when the sizes need more
 * scratch than the static array holds (pa_decode_workspace_bytes() >
 * PA_NOALLOC_SCRATCH_BYTES; with the default work split no single-token
 * call of a supported shape does).
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)17301504)
int pa_decode_noalloc(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                      const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_blocks_per_seq, float scale, void *out, void *stream);

/*
 * pa_decode_multi - attention of q_len new tokens per sequence over the paged
 * cache, causal: new token j of a sequence with context length n (its new
 * tokens included, already written by pa_reshape_and_cache at positions
 * n-q_len .. n-1) attends over positions 0 .. n-q_len+j. This is what a
 * step that verifies speculative tokens in one forward pass, or runs a
 * chunk of a prefill, needs ("vLLM: Anatomy and Mechanisms of
 * High-Throughput LLM Inference", sections "Speculative Decoding" and
 * "Chunked Prefill"; "Inside vLLM", section "Scheduler": the new tokens of a
 * step are not always 1).
 *
 *   q, out   bf16 [num_seqs, q_len, num_q_heads, head_size], 16-byte aligned
 *   q_len    >= 1, with q_len * (num_q_heads / num_kv_heads) <= 256 (any
 *            of the cache's block sizes, 8, 16 or 32): a 64-token prefill
 *            chunk with 4 query heads per KV head, or 7 speculative tokens
 *            (8 new tokens) with 8 or 16. Up to 64 such columns one
 *            wavefront serves a KV head; past 64, a workgroup serves one KV
 *            head with one wavefront per 32 columns, and the same
 *            wavefronts share each block the cache reads.
 * Other arguments, the workspace (size from pa_decode_multi_workspace_bytes)
 * and the errors are those of pa_decode; q_len == 1 is pa_decode. Every
 * context length must be 0 or >= q_len; a new token that would see no
 * position gets a zero output.
 */
int pa_decode_multi(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                    const int32_t *context_lens, int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                    int32_t max_blocks_per_seq, float scale, void *out, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Workspace bytes of pa_decode_multi (as pa_decode_workspace_bytes). */
size_t pa_decode_multi_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t q_len,
                                       int32_t num_q_heads, int32_t max_blocks_per_seq);

/*
 * pa_decode_shared - pa_decode for a batch in which groups of sequences share
 * the leading blocks of their block tables. The outputs of parallel sampling
 * share the prompt's blocks, and beams share their history ("vLLM: Anatomy
 * and Mechanisms of High-Throughput LLM Inference", section "Memory Sharing
 * via Copy-on-Write (CoW)"). Prompts with a common beginning reuse cached
 * blocks (same page, section "Prefix Caching"). Here the shared blocks are
 * read from HBM once for up to 32 / (num_q_heads / num_kv_heads) members of a
 * group, instead of once for each member.
 *
 *   group_starts   int32 [num_groups + 1], device memory. Group g is the
 *                  sequences group_starts[g] .. group_starts[g+1]-1. The
 *                  array must not decrease and must stay within 0..num_seqs.
 *                  Sequences in no group are on their own. If the array
 *                  breaks these rules, no group is formed: every sequence
 *                  reads its own table, as in pa_decode.
 *   shared_blocks  int32 [num_groups], device memory: the number of leading
 *                  table entries the members of group g have in common.
 *   num_groups     0 .. num_seqs. With 0 there is no sharing, and the two
 *                  arrays may be NULL.
 * Which blocks are read:
 *   - Group g's prefix counts only whole blocks that every member fills:
 *     e = min(shared_blocks[g], context_lens[j] / block_size for each
 *     member j), clamped to 0..max_blocks_per_seq.
 *   - Every member reads those e blocks through the table of the group's
 *     first member, and the rest through its own table.
 * When the declaration is true, the result is pa_decode's up to rounding
 * (the sums run in a different order). A false declaration reads the first
 * member's blocks, which is defined and stays in bounds.
 * Limits: num_seqs <= 4096; block_size 8, 16 or 32. The other arguments, layouts and
 * errors are those of pa_decode. The workspace (owned by the caller, or allocated
 * stream-ordered by the call when NULL) has the size that
 * pa_decode_shared_workspace_bytes returns, which is never 0 for
 * num_seqs > 0. Errors: as pa_decode, plus PA_ERR_SHAPE (num_groups outside
 * 0..num_seqs) and PA_ERR_UNSUPPORTED (num_seqs > 4096).
 */
int pa_decode_shared(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                     const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_blocks_per_seq, const int32_t *group_starts, const int32_t *shared_blocks,
                     int32_t num_groups, float scale, void *out, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Workspace bytes of pa_decode_shared (0 on invalid arguments or num_seqs == 0). */
size_t pa_decode_shared_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t max_blocks_per_seq, int32_t num_groups);

/*
 * pa_decode_shared_tree - pa_decode for a batch whose sequences form a tree
 * of shared prefixes, listed depth first, each declaring the leading table
 * entries it holds in common with the sequence before it. Beams hold the
 * prompt in common and, past it, the history of the beam each forked from:
 * after a step, beams that picked the same parent hold every full block of
 * that parent ("vLLM: Anatomy and Mechanisms of High-Throughput LLM
 * Inference", section "Memory Sharing via Copy-on-Write (CoW)"); cached
 * prompt prefixes form such a tree as well (same page, section "Prefix
 * Caching"). Listed depth first (for example sorted by their table rows),
 * the sequences below any node are consecutive, and what sequences i .. k
 * hold in common is the least of the declarations of i+1 .. k. A block is
 * then read from HBM once for each run of up to
 * 32 / (num_q_heads / num_kv_heads) consecutive sequences that hold it,
 * where pa_decode_shared shares only one prefix per group.
 *
 *   shared_prev  int32 [num_seqs], device memory: shared_prev[i] is the
 *                number of leading table entries that sequence i has in
 *                common with sequence i - 1. shared_prev[0] is ignored.
 * Which blocks are read:
 *   - Sequence i > 0 shares e_i = min(shared_prev[i],
 *     context_lens[i] / block_size, context_lens[i-1] / block_size) blocks
 *     with sequence i - 1 (whole blocks both fill), clamped to
 *     0..max_blocks_per_seq; negative declarations count as 0.
 *   - Sharing is by 16-token chunks of those blocks: with 8-token blocks an
 *     odd e_i leaves its last shared block to sequence i's own reads.
 *   - Each sequence reads the chunks it does not share with the one before
 *     it through its own table, for itself and for every later sequence
 *     whose shared chunks reach them without a break.
 * When every declaration is true, the result is pa_decode's up to rounding
 * (the sums run in a different order). A false declaration makes the
 * outputs of the sequences after it unspecified; every read still goes
 * through a table row of the batch, with the usual clamping of block ids.
 * Limits, other arguments, layouts and errors are those of pa_decode_shared,
 * plus PA_ERR_NULL for shared_prev == NULL when num_seqs > 0. The workspace
 * has the size pa_decode_shared_tree_workspace_bytes returns.
 */
int pa_decode_shared_tree(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                          const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                          int32_t max_blocks_per_seq, const int32_t *shared_prev, float scale, void *out,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of pa_decode_shared_tree (0 on invalid arguments or num_seqs == 0). */
size_t pa_decode_shared_tree_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                                             int32_t max_blocks_per_seq);

/*
 * pa_share_plan, pa_decode_shared_planned - the two halves of
 * pa_decode_shared / pa_decode_shared_tree, for a model whose layers all
 * decode the same batch. The sharing-aware call first builds a plan (which
 * blocks each segment of sequences reads, from the context lengths and the
 * declaration alone), then decodes on it. The plan holds nothing of q, the
 * caches or the output, so within a step it is the same for every layer:
 * build it once with pa_share_plan, then call pa_decode_shared_planned per
 * layer. Each planned call gives the result of the one-call form bit for bit.
 *
 *   plan          device memory of at least pa_share_plan_bytes(...) bytes,
 *                 16-byte aligned, owned by the caller. pa_share_plan writes
 *                 it (stream-ordered); it needs no initialisation.
 *   pa_share_plan takes the arguments of pa_decode_shared (group form:
 *                 group_starts, shared_blocks, num_groups) or, when
 *                 shared_prev is not NULL, of pa_decode_shared_tree (chain
 *                 form; the group arguments are then ignored), with the same
 *                 rules and clamps. context_lens is read once, by the plan.
 *   pa_decode_shared_planned takes q, block_tables, scale, out and a
 *                 workspace of pa_decode_shared_planned_workspace_bytes(...)
 *                 (or NULL: allocated stream-ordered by the call), as
 *                 pa_decode_shared does.
 * The plan is valid for the cache descriptor's num_kv_heads and block_size,
 * num_seqs, num_q_heads and max_blocks_per_seq it was made with, and for the
 * context lengths it read; with other sizes or lengths the output is
 * unspecified (every access stays inside the arrays the call is given).
 * Calls that share a plan may overlap; calls that share a workspace may not.
 * Errors: those of pa_decode_shared, plus PA_ERR_NULL (plan NULL) and
 * PA_ERR_WORKSPACE (plan smaller than pa_share_plan_bytes or not 16-byte
 * aligned).
 */
size_t pa_share_plan_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                           int32_t max_blocks_per_seq);

int pa_share_plan(const pa_kv_cache *cache, const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                  int32_t max_blocks_per_seq, const int32_t *group_starts, const int32_t *shared_blocks,
                  int32_t num_groups, const int32_t *shared_prev, void *plan, size_t plan_bytes, void *stream);

size_t pa_decode_shared_planned_workspace_bytes(const pa_kv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                                                int32_t max_blocks_per_seq);

int pa_decode_shared_planned(const pa_kv_cache *cache, const void *q, const int32_t *block_tables,
                             int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq, const void *plan,
                             float scale, void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_reshape_and_cache - write each new token's K and V into its physical
 * slot before attention runs (the slot the block manager assigned on demand:
 * "vLLM: Anatomy and Mechanisms", section "Block-Level Management"; the
 * decode step that follows sees every earlier token cached: "Inside vLLM",
 * section "Scheduler").
 *
 *   k, v          bf16 [num_tokens, num_kv_heads, head_size], contiguous,
 *                 16-byte aligned
 *   slot_mapping  int64 [num_tokens]; slot = block*block_size + offset. A
 *                 negative slot (padding) or a slot >= num_blocks*block_size
 *                 is skipped.
 *                 Slots must be distinct (otherwise which token wins is
 *                 unspecified).
 * The copy is bit-exact. num_tokens == 0 is a no-op.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (num_tokens < 0), PA_ERR_UNSUPPORTED,
 * PA_ERR_HIP.
 */
int pa_reshape_and_cache(const pa_kv_cache *cache, const void *k, const void *v,
                         const int64_t *slot_mapping, int32_t num_tokens, void *stream);

/*
 * pa_copy_blocks - copy-on-write of diverging blocks ("vLLM: Anatomy and
 * Mechanisms", section "Memory Sharing via Copy-on-Write (CoW)": only the
 * block where beams diverge is copied).
 *
 *   src_dst_pairs int64 [num_pairs][2], device memory: block dst becomes a
 *                 bit copy of block src, for K and for V. Destinations must
 *                 be distinct and never also a source (a CoW destination is
 *                 a fresh block); otherwise the result is unspecified. A pair
 *                 with an index outside [0, num_blocks) is skipped.
 * num_pairs == 0 is a no-op.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (num_pairs < 0), PA_ERR_UNSUPPORTED,
 * PA_ERR_HIP.
 */
int pa_copy_blocks(const pa_kv_cache *cache, const int64_t *src_dst_pairs, int32_t num_pairs,
                   void *stream);

/* Directions of pa_swap_blocks. */
enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 };

/*
 * pa_swap_blocks - move whole blocks between the device cache and a host
 * cache, for preemption by swapping: a preempted request's KV blocks go to
 * CPU RAM and come back when it resumes ("vLLM: Anatomy and Mechanisms of
 * High-Throughput LLM Inference", section "Preemption and Recovery";
 * "vLLM Internals", section "The Block Manager").
 *
 *   host_k, host_v   bf16 [host_num_blocks, block_size, num_kv_heads, head_size],
 *                    contiguous, in pinned host memory (hipHostMalloc, or
 *                    a pinned torch tensor); owned by the caller, who
 *                    guarantees host_num_blocks blocks of each. The library
 *                    asks the HIP runtime for their device address and
 *                    returns PA_ERR_UNSUPPORTED for memory it does not know
 *                    as pinned host memory.
 *   src_dst_pairs    int64 [num_pairs][2], device memory. PA_SWAP_OUT: host
 *                    block dst becomes a bit copy of device block src;
 *                    PA_SWAP_IN: device block dst becomes a bit copy of host
 *                    block src. K and V both. Destinations must be distinct;
 *                    a pair with an index outside its side's pool is
 *                    skipped.
 *   direction        PA_SWAP_OUT or PA_SWAP_IN
 * Asynchronous on `stream`; the host array is complete (swap out) or may be
 * reused (swap in) once the stream has reached the call. num_pairs == 0 is a
 * no-op.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (num_pairs < 0, host_num_blocks < 0, bad
 * direction), PA_ERR_UNSUPPORTED (see pa_kv_cache; host memory not pinned),
 * PA_ERR_HIP.
 */
int pa_swap_blocks(const pa_kv_cache *cache, void *host_k, void *host_v, int64_t host_num_blocks,
                   const int64_t *src_dst_pairs, int32_t num_pairs, int32_t direction, void *stream);

/* Text of the last error on this thread ("" after a successful call). */
const char *pa_last_error(void);

/*
 * Measurement helper, not part of the decode path: copy `bytes` bytes (a
 * multiple of 16, both pointers 16-byte aligned) with plain 16-byte vector
 * loads and stores. Used to calibrate hardware byte counters and to measure
 * achievable HBM bandwidth.
 */
int pa_probe_copy(void *dst, const void *src, size_t bytes, void *stream);

/*
 * Measurement helper, not part of the decode path: read `bytes` bytes of
 * device memory at `src` (a multiple of 16, 16-byte aligned) with plain
 * 16-byte vector loads and write one folded 32-bit word per thread to the
 * device buffer `sink` (at least pa_probe_read_sink_bytes() bytes), so that
 * the achievable HBM read bandwidth can be timed. Errors: PA_ERR_NULL,
 * PA_ERR_SHAPE (size or alignment), PA_ERR_WORKSPACE (sink too small),
 * PA_ERR_HIP.
 */
size_t pa_probe_read_sink_bytes(void);
int pa_probe_read(const void *src, size_t bytes, void *sink, size_t sink_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
