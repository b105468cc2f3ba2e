/*
 * pa.h -- C ABI of the paged-KV attention step for AMD Instinct MI355X (gfx950).
 *
 * One continuous-batching step of a decoder layer, as the pages describe it:
 *   1. the new tokens' K/V are scattered into a block pool through a slot
 *      mapping (slot = physical_block * block_size + offset), and
 *   2. GQA attention runs over a flattened, padding-free batch that mixes
 *      decode tokens and prefill chunks, reading history through a per-request
 *      block table with the causal mask at absolute positions.
 *
 * Sources (web pages; section names as printed):
 *   [P1] "AI Infra入门干货总结：大模型是如何高效推理的" (joto.ai): sections
 *        "连续批处理 (Continuous Batching)", "Paged Attention",
 *        "Attention Module (以标准GQA + RoPE为例)", "总结".
 *   [P4] "Chunked Prefill 与 Preemption" (llm-glossary.tokens-kit.com):
 *        section "Chunked Prefill：改变调度粒度，不改变 causal 结果", equation M_{i,j}.
 *   [P5] "显存与调度" (aaai.latere.ai, chapter 32): sections "从保留词元到物理块",
 *        "块表消除连续内存要求".
 *
 * Conventions for every entry point
 *   - The caller owns every buffer.  The library keeps no pointer after a call
 *     returns and allocates no device memory; pa_attention takes a
 *     caller-provided workspace.
 *   - "device" pointers are HIP device memory of the current device; "host"
 *     pointers are ordinary host memory, read before the call returns.
 *   - Calls taking a stream enqueue work on it (NULL = the null stream) and
 *     return without synchronising.  pa_write_kv for a layer must be enqueued
 *     before pa_attention of that layer: attention reads the step's own K/V
 *     back from the cache ([P1] "Attention Module": the prompt's K/V are first
 *     written by the cache-write kernel, then read through the block table).
 *   - Every argument that can be checked on the host is checked before any
 *     work is enqueued; a failing check returns a status, sets
 *     pa_last_error() and enqueues nothing.  Nothing aborts or throws across
 *     the ABI.  Index values that live only in device memory (block ids, slot
 *     values) are not checked on the fast path: the kernels clamp every block
 *     id into the pool, so bad indices give wrong numbers but no out-of-bounds
 *     access; pa_validate_metadata checks host copies of them exactly.
 *   - Tensors are dense and row-major with the shapes given below.
 *   - Support matrix: head_dim in {64, 128}; block_size a positive multiple of
 *     16; num_heads % num_kv_heads == 0 with num_heads / num_kv_heads in
 *     {1, 2, 4, 8}; dtype PA_F32 or PA_BF16, shared by query, key, value,
 *     caches and output.  Anything else returns PA_ERR_UNSUPPORTED.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL_PTR = 1,
  PA_ERR_BAD_SHAPE = 2,
  PA_ERR_BAD_DTYPE = 3,
  PA_ERR_UNSUPPORTED = 4,
  PA_ERR_OUT_OF_RANGE = 5,
  PA_ERR_DUPLICATE_SLOT = 6,
  PA_ERR_INCONSISTENT_METADATA = 7,
  PA_ERR_WORKSPACE_TOO_SMALL = 8,
  PA_ERR_HIP = 9,
  PA_ERR_BAD_STATE = 10   /* a stateful object (scheduler) called out of order */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* ABI version of the loaded library (PA_ABI_VERSION it was built with). */
int pa_abi_version(void);

/* Static, never-NULL name of a status code ("PA_OK", ...; "PA_UNKNOWN" for
 * values outside the enum). */
const char* pa_status_str(int status);

/* Detail of the last failing call on the calling thread ("" if none).  The
 * string stays valid until the next library call on this thread. */
const char* pa_last_error(void);

/*
 * pa_build_step_metadata -- host-side step metadata for a flattened batch.
 *
 * [P1] "连续批处理": a step schedules, per request, the tokens between
 * num_computed_tokens and its current length, and all scheduled tokens form
 * one flattened batch; [P1] "Attention Module" ("特别注意"): cumulative
 * sequence lengths isolate requests inside that batch; [P1] "Paged
 * Attention": token position p of request r is stored at
 * block_table[r][p / block_size] * block_size + p % block_size.
 *
 *   h_query_lens        host int32 [R]   tokens scheduled for request r (>= 0)
 *   h_num_computed      host int32 [R]   tokens of r already in the cache (>= 0)
 *   h_block_table       host int32 [R, max_blocks_per_req] physical block ids;
 *                       entry j must be valid for j < ceil(seq_len / block_size)
 *   h_query_start_loc   host int32 [R + 1] out: exclusive prefix sum of query_lens
 *   h_seq_lens          host int32 [R]     out: num_computed + query_lens
 *   h_slot_mapping      host int64 [slot_capacity] out: flat slot of every
 *                       scheduled token, in flattened order
 * Returns PA_ERR_OUT_OF_RANGE if a needed block-table entry is outside
 * [0, num_blocks) or a sequence needs more than max_blocks_per_req blocks,
 * PA_ERR_BAD_SHAPE if the tokens exceed slot_capacity or a count is negative.
 * Outputs are unspecified on error.
 */
pa_status pa_build_step_metadata(const int32_t* h_query_lens, const int32_t* h_num_computed,
                                 int32_t R, const int32_t* h_block_table,
                                 int32_t max_blocks_per_req, int32_t block_size,
                                 int32_t num_blocks, int32_t* h_query_start_loc,
                                 int32_t* h_seq_lens, int64_t* h_slot_mapping,
                                 int64_t slot_capacity);

/*
 * pa_compute_slot_mapping -- the same slot mapping, computed on the device.
 *
 * [P1] "Paged Attention": token i of request r (flattened index
 * query_start_loc[r] + i) is at position p = num_computed_tokens[r] + i and
 * goes to slot block_table[r][p / block_size] * block_size + p % block_size.
 *
 *   slot_mapping        device int64 [T] (written)
 *   block_table         device int32 [R, max_blocks_per_req]
 *   query_start_loc     device int32 [R + 1]
 *   num_computed_tokens device int32 [R]
 * A token whose block-table entry lies outside [0, num_blocks), or whose
 * position is past the end of its block-table row, gets slot -1 (pa_write_kv
 * then writes nothing for it; pa_validate_metadata reports the cause).
 * Tokens outside every request's range are left untouched.
 */
pa_status pa_compute_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                                  int32_t max_blocks_per_req, const int32_t* query_start_loc,
                                  const int32_t* num_computed_tokens, int32_t R, int64_t T,
                                  int32_t num_blocks, int32_t block_size, void* stream);

/*
 * pa_write_kv -- scatter the step's new K/V rows into the paged cache.
 *
 * [P1] "Paged Attention" (slot_idx = block_idx * block_size + block_offset;
 * block = slot / block_size, offset = slot % block_size) and "Attention
 * Module" (the new K/V are scattered into the paged cache by slot mapping).
 *
 *   key, value          device [T, num_kv_heads, head_dim]
 *   key_cache,
 *   value_cache         device [num_blocks, block_size, num_kv_heads, head_dim],
 *                       written in place: row t goes to
 *                       cache[slot / block_size][slot % block_size]
 *   slot_mapping        device int64 [T]; a negative slot writes nothing
 * The copy is exact (bit-for-bit).  Slots must be distinct and below
 * num_blocks * block_size; a slot at or past the end of the pool is skipped on
 * the fast path (pa_validate_metadata reports it).  T == 0 is a no-op.
 */
pa_status pa_write_kv(const void* key, const void* value, void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int64_t T, int32_t num_blocks,
                      int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                      pa_dtype dtype, void* stream);

/*
 * pa_rope_write_kv -- rotary position embedding of Q and K fused with the
 * cache write.
 *
 * [P1] "Attention Module (以标准GQA + RoPE为例)": Q and K of a token are
 * multiplied by a block-diagonal rotation whose angles depend on the token's
 * position; the rotation is applied elementwise from a table cos_sin_cache
 * [max_position_embeddings, rotary_dim] prepared once, whose row p holds the
 * cos of the rotary_dim / 2 angles of position p followed by their sin; then
 * K and V are scattered into the paged cache by slot_mapping.  For angle
 * column i and coordinate pair (a, b): x_a' = x_a cos_i - x_b sin_i,
 * x_b' = x_b cos_i + x_a sin_i.  neox_style = 1 pairs (i, i + rotary_dim/2),
 * neox_style = 0 pairs (2i, 2i + 1); coordinates at or past rotary_dim are
 * not rotated.
 *
 *   query               device [T, num_heads, head_dim], rotated in place
 *   key, value          device [T, num_kv_heads, head_dim] (read only; the
 *                       rotated K is written to the cache, not back to key)
 *   key_cache,
 *   value_cache         device [num_blocks, block_size, num_kv_heads, head_dim];
 *                       slot s gets the rotated K row and the V row of its
 *                       token, exactly as pa_write_kv would write them
 *   slot_mapping        device int64 [T]; a negative slot writes nothing to
 *                       the caches (its query row is still rotated)
 *   positions           device int64 [T] absolute position of each token
 *                       (num_computed_tokens + i); values outside
 *                       [0, max_position) are clamped into it
 *   cos_sin_cache       device float32 [max_position, rotary_dim]
 *   rotary_dim          positive multiple of 16, at most head_dim
 * Arithmetic is fp32, rounded once to dtype.  Slots must be distinct and
 * below num_blocks * block_size (past the pool: skipped).  T == 0 is a no-op.
 * pa_attention of the layer must be enqueued after this call.
 */
pa_status pa_rope_write_kv(void* query, const void* key, const void* value, void* key_cache,
                           void* value_cache, const int64_t* slot_mapping, const int64_t* positions,
                           const float* cos_sin_cache, int32_t max_position, int32_t rotary_dim,
                           int32_t neox_style, int64_t T, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t num_blocks, int32_t block_size,
                           pa_dtype dtype, void* stream);

/*
 * pa_copy_blocks -- copy whole cache blocks between pools of one block layout.
 *
 * Serves two block movements the pages describe: copy-on-write of a shared,
 * partly filled block before a request writes into it ([P5] "显存与调度",
 * "共享前缀会改变块的所有权": a writable shared block needs copy-on-write; the
 * scheduler of pa_sched.h lists the pairs), and swap-out / swap-in of a
 * preempted request's blocks between the device cache and a pinned host
 * pool ([P2] "vLLM 抢占机制源码精读", section "Swap 模式"; [P4] "Chunked Prefill
 * 与 Preemption": the swap round trip moves the payload out and back).
 *
 *   src_pools, dst_pools  num_pools pools each, pool k at base + k * stride
 *                         bytes (e.g. the 2L per-layer K and V caches of a
 *                         model); device memory, or pinned host memory from
 *                         hipHostMalloc (read or written over the host link)
 *   block_pairs           device int32 [num_pairs, 2]: (source block,
 *                         destination block); pair i copies block_bytes bytes
 *                         from source block of every source pool to the
 *                         destination block of the matching destination pool
 *   src_num_blocks,
 *   dst_num_blocks        blocks per pool; pairs outside them are skipped
 *   block_bytes           bytes of one block (block_size * num_kv_heads *
 *                         head_dim * element size), a multiple of 16
 * Destination blocks must be distinct and must not be a source of the same
 * call (else the result is undefined).  The copy is exact.  Enqueued on
 * stream; a plan's copies must be enqueued before its cache write.  A copy
 * that crosses the host link (either side pinned host memory, as
 * hipPointerGetAttributes reports it) runs on at most 64 workgroups; it still
 * occupies the memory path of the compute units for the whole transfer, so
 * swaps beside a running step belong on the copy engines (pa_swap_blocks).
 * Returns PA_ERR_BAD_SHAPE for a pool pointer that is neither device memory
 * nor pinned host memory.
 */
pa_status pa_copy_blocks(const void* src_pools, void* dst_pools, const int32_t* block_pairs,
                         int32_t num_pairs, int32_t num_pools, int64_t src_pool_stride,
                         int64_t dst_pool_stride, int32_t src_num_blocks, int32_t dst_num_blocks,
                         int64_t block_bytes, void* stream);

/*
 * pa_swap_blocks -- swap-out / swap-in of whole cache blocks on the GPU's
 * copy engines.
 *
 * [P2] "vLLM 抢占机制源码精读", section "Swap 模式": a preempted request's
 * blocks are moved to host memory and back asynchronously by the cache
 * engine, before the model's kernels run; [P4] "Chunked Prefill 与
 * Preemption": the swap round trip moves the payload out and back, bounded
 * by twice the payload over the host-link bandwidth.
 *
 *   src_pools, dst_pools  num_pools pools each, pool k at base + k * stride
 *                         bytes (the 2L per-layer K and V caches of a model);
 *                         device memory or pinned host memory (any pairing)
 *   h_block_pairs         HOST int32 [num_pairs, 2]: (source block,
 *                         destination block); pair i copies block_bytes bytes
 *                         from the source block of every source pool to the
 *                         destination block of the matching destination pool
 *   block_bytes           bytes of one block of one pool
 * Each run of consecutive pairs whose source and destination blocks both
 * advance by one becomes one 2-D asynchronous copy (width = run * block_bytes,
 * height = num_pools, pitches = the pool strides), enqueued on stream in pair
 * order: the copy engines move the data, so the compute units and their memory
 * path stay with the kernels of a step running on another stream (order the
 * two with events: the step must not write blocks being swapped out nor read
 * blocks being swapped in).  The copy is exact; nothing is allocated.
 * Checked on the host before anything is enqueued: pointers, sizes, strides
 * (>= a pool when num_pools > 1), every block id within its pool
 * (PA_ERR_OUT_OF_RANGE) and distinct destination blocks
 * (PA_ERR_DUPLICATE_SLOT).  A HIP error while enqueueing returns PA_ERR_HIP;
 * the copies enqueued before it stay enqueued.
 */
pa_status pa_swap_blocks(const void* src_pools, void* dst_pools, const int32_t* h_block_pairs,
                         int32_t num_pairs, int32_t num_pools, int64_t src_pool_stride,
                         int64_t dst_pool_stride, int32_t src_num_blocks, int32_t dst_num_blocks,
                         int64_t block_bytes, void* stream);

/*
 * pa_attention_workspace_bound -- bytes of device workspace that cover every
 * step within the given limits, so that a server can allocate the workspace
 * once ([P1] "Paged Attention": the step's tables are sized by static maxima,
 * block_table being [max_num_reqs, max_num_blocks_per_req]).
 *
 *   max_num_reqs     most requests in one step (R)
 *   max_num_tokens   most flattened query rows in one step (T)
 *   max_seq_len      longest seq_len of any request in a step
 * Returns a size >= pa_attention_workspace_size(...) for every step with
 * R <= max_num_reqs, T <= max_num_tokens and every seq_len <= max_seq_len,
 * for the given geometry on the current device (with the tuning overrides of
 * pa_set_tuning in force at the time of the call).  The bound follows from
 * the partition and segment rules (it is not a measured maximum) and is
 * largest for long prefill chunks deep into long prompts, whose key segments
 * each need their own partial results.  Returns 0 and sets pa_last_error()
 * for unsupported geometry or negative limits.
 */
size_t pa_attention_workspace_bound(int32_t max_num_reqs, int64_t max_num_tokens,
                                   int32_t max_seq_len, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, pa_dtype dtype);

/*
 * pa_attention_workspace_size -- bytes of device workspace pa_attention needs
 * for this step (plan tables plus split-K partial results).  Takes the same
 * host mirrors pa_attention plans from; returns 0 and sets pa_last_error() if
 * they are invalid.  The size depends on these arguments and on the current
 * device (its compute units and the split-K kernel's occupancy set the
 * partition length), so query it with the device current that pa_attention
 * will run on.
 */
size_t pa_attention_workspace_size(const int32_t* h_query_start_loc, const int32_t* h_seq_lens,
                                   int32_t R, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, pa_dtype dtype);

/*
 * pa_attention -- GQA attention of one step over the paged cache.
 *
 * Definition ([P1] "Attention Module"; [P4] equation M_{i,j}; [P5]
 * "块表消除连续内存要求"): for request r with n_r = query_start_loc[r+1] -
 * query_start_loc[r] query rows, seq_len L_r and num_computed c_r, query row
 * i (flattened index query_start_loc[r] + i) sits at absolute position c_r + i;
 * query head h uses kv head h / (num_heads / num_kv_heads); its output is
 *   softmax_j(scale * <q, K_r[j]>) . V_r[j]  over keys j = 0 .. c_r + i,
 * where K_r/V_r are the request's first L_r positions gathered through
 * block_table[r].  A request with n_r == 1 is a decode row (it sees all L_r
 * keys); n_r > 1 is a prefill chunk.  Requests never interact.
 *
 *   out                 device [T, num_heads, head_dim] (written; rows of
 *                       requests with n_r == 0 do not exist)
 *   query               device [T, num_heads, head_dim]
 *   key_cache,
 *   value_cache         device [num_blocks, block_size, num_kv_heads, head_dim]
 *   block_table         device int32 [R, max_blocks_per_req]
 *   query_start_loc     device int32 [R + 1]
 *   seq_lens            device int32 [R]
 *   num_computed_tokens device int32 [R] (must equal seq_lens - query lens)
 *   h_query_start_loc,
 *   h_seq_lens          host copies of the two arrays above; used only to size
 *                       the launch and check the workspace, never to compute
 *                       results.  They must equal the device arrays.
 *   scale               softmax scale (1/sqrt(head_dim) for standard attention)
 *   workspace           device buffer of at least
 *                       pa_attention_workspace_size(...) bytes, 256-byte
 *                       aligned; contents on entry are ignored
 * Requirements checked on the host: query_start_loc[0] == 0, non-decreasing,
 * query_start_loc[R] == T; 0 <= n_r <= L_r; L_r <= max_blocks_per_req *
 * block_size.  The result does not depend on request order or on which
 * physical blocks hold the data.
 */
pa_status pa_attention(void* out, const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_table,
                       int32_t max_blocks_per_req, const int32_t* query_start_loc,
                       const int32_t* seq_lens, const int32_t* num_computed_tokens,
                       const int32_t* h_query_start_loc, const int32_t* h_seq_lens, int32_t R,
                       int64_t T, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t num_blocks, int32_t block_size, float scale, pa_dtype dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_attention_plan / pa_attention_run -- pa_attention in two calls, so that
 * a step is planned once and attended layer by layer.
 *
 * [P1] "Paged Attention": slot_mapping and block_table have no layer
 * dimension -- every layer of a step uses the same metadata -- so the work
 * plan of a step is the same for all its layers; only the query, the output
 * and the layer's caches change.
 *
 * pa_attention_plan checks the step exactly as pa_attention does, enqueues
 * the device planner on stream (it writes the work tables into the
 * workspace) and fills *plan on the host.  pa_attention_run enqueues the
 * attention of one layer with that plan.  pa_attention(...) is the same as
 * pa_attention_plan followed by one pa_attention_run on the same stream.
 *
 *   plan   caller-owned record; its contents are private to the library (copy
 *          it only as a whole).  It holds the device pointers block_table,
 *          query_start_loc, seq_lens, num_computed_tokens and workspace given
 *          to pa_attention_plan: they must stay valid and unchanged until the
 *          last pa_attention_run with this plan has executed.
 * Every pa_attention_run of a plan must be ordered after its
 * pa_attention_plan on the device (same stream, or joined by an event), and
 * no other plan may be written into the same workspace until the runs have
 * executed; runs that share a workspace must not overlap each other (they
 * reuse its partial-result space), so enqueue them on one stream.  The
 * arguments of pa_attention_plan mean what they mean for pa_attention; those
 * of pa_attention_run are the per-layer ones (out, query, key_cache,
 * value_cache with the planned geometry, and scale).
 */
typedef struct pa_step_plan { int64_t words[48]; } pa_step_plan;

pa_status pa_attention_plan(pa_step_plan* plan, const int32_t* block_table,
                            int32_t max_blocks_per_req, const int32_t* query_start_loc,
                            const int32_t* seq_lens, const int32_t* num_computed_tokens,
                            const int32_t* h_query_start_loc, const int32_t* h_seq_lens,
                            int32_t R, int64_t T, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t num_blocks, int32_t block_size,
                            pa_dtype dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

pa_status pa_attention_run(const pa_step_plan* plan, void* out, const void* query,
                           const void* key_cache, const void* value_cache, float scale,
                           void* stream);

/*
 * pa_set_tuning / pa_get_tuning -- overrides of the library's own kernel and
 * partition choices, for tests and measurements.
 *
 * Every knob is 0 by default, which is the product behaviour; results differ
 * only by rounding between settings.  The setting is process-wide and read
 * when a step is planned (pa_attention, pa_attention_plan, the workspace
 * queries), so set it before those calls and not while other threads plan.
 *   PA_TUNE_DECODE_KERNEL       1: vector split-K kernel, 2: matrix-core
 *                               split-K kernel (bf16 with 4 or 8 q heads per
 *                               kv head; elsewhere the vector kernel runs)
 *   PA_TUNE_DECODE_Q_PLACEMENT  1: query rows in registers, 2: in LDS
 *                               (vector split-K kernel)
 *   PA_TUNE_SPLIT_KEYS          n > 0: split-K partition length, rounded up
 *                               to the partition unit and capped at 64 blocks
 *   PA_TUNE_SPLIT_RULE          1: the device-independent partition rule
 *                               (about 32 waves per compute unit) instead of
 *                               the occupancy-based one
 *   PA_TUNE_CHUNK_SEGMENT       n > 0: chunk key-segment length (rounded up
 *                               to 64, capped at the kernel's limit)
 *   PA_TUNE_CHUNK_PATH          1: every multi-token request takes the
 *                               split-K path instead of the matrix-core
 *                               chunk kernel
 *   PA_TUNE_DECODE_STAGING      1: the split-K kernels' per-head form (one
 *                               wavefront per kv head streaming its own rows
 *                               through registers) instead of the default
 *                               whole-block form (bf16, head_dim 128, 1/2/4/8
 *                               kv heads: one workgroup per item staging whole
 *                               16-token slabs of all kv heads in LDS)
 * pa_set_tuning returns PA_ERR_BAD_SHAPE for an unknown knob or a negative
 * value; pa_get_tuning returns -1 for an unknown knob.
 */
typedef enum pa_tuning_knob {
  PA_TUNE_DECODE_KERNEL = 0,
  PA_TUNE_DECODE_Q_PLACEMENT = 1,
  PA_TUNE_SPLIT_KEYS = 2,
  PA_TUNE_SPLIT_RULE = 3,
  PA_TUNE_CHUNK_SEGMENT = 4,
  PA_TUNE_CHUNK_PATH = 5,
  PA_TUNE_DECODE_STAGING = 6,
  PA_TUNE_COUNT = 7
} pa_tuning_knob;

pa_status pa_set_tuning(int32_t knob, int32_t value);
int32_t pa_get_tuning(int32_t knob);

/*
 * pa_attention_noalloc -- pa_attention without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, checks and results as pa_attention, minus workspace and
 * workspace_bytes: the step's plan tables and partial results go to a static
 * device array of PA_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * every GPU it runs on until the process ends.  The call allocates nothing.
 * A step whose workspace (pa_attention_workspace_size) exceeds
 * PA_NOALLOC_SCRATCH_BYTES is refused with PA_ERR_WORKSPACE_TOO_SMALL before
 * anything is enqueued.  Nothing in the scratch needs clearing between calls
 * (every table is rewritten by each call's planner).  All calls on one GPU
 * share its scratch: calls that overlap on one GPU (different streams or
 * threads without ordering) race and give wrong results; order them on one
 * stream.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

pa_status pa_attention_noalloc(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_table,
                               int32_t max_blocks_per_req, const int32_t* query_start_loc,
                               const int32_t* seq_lens, const int32_t* num_computed_tokens,
                               const int32_t* h_query_start_loc, const int32_t* h_seq_lens,
                               int32_t R, int64_t T, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t num_blocks, int32_t block_size,
                               float scale, pa_dtype dtype, void* stream);

/*
 * pa_set_profiling_events -- optional per-kernel timing hook (tests and
 * benchmarks).
 *
 * events: host array of n_events == 5 hipEvent_t handles created by the
 * caller on the current device, or NULL / n_events == 0 to disable.  While set
 * on the calling thread, every pa_attention call records, on its stream,
 * events[0] before its first launch and events[1], [2], [3], [4] after the
 * plan, row-wise split-K, chunk and merge launches (pa_attention_plan records
 * events[0] and [1]; pa_attention_run records events[1] before its first
 * launch, then [2], [3], [4]).  The library copies the handles; the caller
 * keeps ownership of the events.
 */
pa_status pa_set_profiling_events(void* const* events, int32_t n_events);

/*
 * pa_validate_metadata -- exact host-side check of a step's metadata (for
 * tests and debugging; O(R * max_blocks + T)).
 *
 * Checks, in order: pointers and sizes; query_start_loc[0] == 0, monotone,
 * query_start_loc[R] == T; seq_lens[r] == num_computed[r] + n_r; every
 * sequence fits its block-table row; every block-table entry a sequence needs
 * lies in [0, num_blocks); when h_slot_mapping is not NULL, every slot is
 * negative or below num_blocks * block_size (else PA_ERR_OUT_OF_RANGE),
 * every non-negative slot equals the block-table formula for its token
 * (else PA_ERR_INCONSISTENT_METADATA) and no two tokens share a slot
 * (else PA_ERR_DUPLICATE_SLOT).
 */
pa_status pa_validate_metadata(const int32_t* h_query_start_loc, const int32_t* h_seq_lens,
                               const int32_t* h_num_computed, const int32_t* h_block_table,
                               int32_t max_blocks_per_req, const int64_t* h_slot_mapping,
                               int32_t R, int64_t T, int32_t num_blocks, int32_t block_size);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
