/*
 * pa_sched.h -- C ABI of the host-side continuous-batching scheduler and
 * paged block allocator that produce the attention step's inputs
 * (query lengths, computed counts and block tables).
 *
 * Sources (web pages; section names as printed):
 *   [P1] "AI Infra入门干货总结：大模型是如何高效推理的": "连续批处理"
 *        (num_computed_tokens / num_tokens, the step schedules the difference
 *        within a token budget), "附4" (recompute preemption when blocks run
 *        out; no admission in a step that preempted).
 *   [P2] "vLLM 抢占机制源码精读": "抢占的触发条件", "Recompute 模式" (victim
 *        from the tail of the running queue, self-preemption when alone,
 *        preempted requests go to the front of the waiting queue),
 *        "人工抢占测试" (a hook that makes the free-block check fail).
 *   [P5] "显存与调度" (ch. 32): "分配是词元计划的一部分" (Delta q_i =
 *        ceil((T_i + s_i)/B) - ceil(T_i/B); reserve, execute, commit or roll
 *        back; q_free + q_reserved + q_committed = q_capacity),
 *        "分块预填充共享每轮预算" (token budget), "同时验证分配器与调度器"
 *        (the metrics below).
 *
 * Behaviour, per step:
 *   pa_sched_schedule plans a step: running requests in FCFS order each get
 *   min(remaining tokens, chunk, budget left) tokens; their new blocks are
 *   reserved from the front of the free list; when a request's blocks do not
 *   fit, the running request at the tail is preempted by recompute (all its
 *   blocks released, computed tokens reset to 0, it goes to the front of the
 *   waiting queue), or the request itself if it is the last; if nothing was
 *   preempted, waiting requests are admitted in order while a sequence slot,
 *   budget and their blocks are available.  Then exactly one of
 *   pa_sched_commit (the step ran: reservations become committed, computed
 *   counts advance, a request whose computed tokens reach its known tokens
 *   samples one token and finishes after output_len tokens, releasing its
 *   blocks) or pa_sched_rollback (the step failed: the plan's reservations
 *   return to the free list and the requests it admitted go back to the
 *   front of the waiting queue; preemptions are not undone).
 *   pa_sched_cancel may be called at any time; it releases every block the
 *   request holds and drops it from a pending plan.
 * Released blocks go to the back of the free list.  All randomness is an
 * input: the initial free-list order and the uniform draws the
 * artificial-preemption hook consumes (one per free-block check while armed).
 *
 * Shared blocks ([P5] "共享前缀会改变块的所有权", figure 32.2): every block has a
 * reference count; a request that stops using a block (finish, preemption,
 * cancel, rollback) decrements it and only a block at 0 leaves: to the back
 * of the free list, or -- if the prefix index holds it -- into the evictable
 * set (cached state, still committed) in release order.  A request admitted
 * with nothing computed attaches the longest run of its leading block keys
 * found in the index (at most floor((tokens - 1) / block_size) blocks, so a
 * token is always computed and no write lands in a shared full block) and
 * starts after it; after each committed step a request offers its full
 * prompt blocks to the index.  When free blocks run short the least recently
 * released cached blocks are evicted before anything is preempted.  A request
 * about to write into a partly filled block others also reference takes a
 * fresh block instead, drops its reference to the old one, and the plan
 * lists the copy (old -> new) that must run, on every layer's K and V cache,
 * before the step's cache write (copy-on-write); rollback undoes it.
 *
 * Conventions: every pointer is host memory; the library copies what it
 * keeps.  A pa_sched object is not thread-safe.  Failing calls return a
 * status and leave the object unchanged; the detail is in
 * pa_sched_last_error() (thread-local).  Calling schedule twice without a
 * commit or rollback, or commit/rollback without a plan, returns
 * PA_ERR_BAD_STATE.
 */
#ifndef PA_SCHED_H_
#define PA_SCHED_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_sched pa_sched;

typedef struct pa_sched_config {
  int32_t num_blocks;              /* pool capacity q_capacity */
  int32_t block_size;              /* tokens per block, > 0 */
  int32_t max_num_seqs;            /* running requests per step */
  int32_t max_num_batched_tokens;  /* token budget K per step */
  int32_t chunk;                   /* prefill tokens per request per step */
  const int32_t* block_order;      /* [num_blocks] initial free list: a permutation of 0..num_blocks-1 */
  double hook_prob;                /* artificial preemption: fail a free-block check when draw < prob */
  int32_t hook_max;                /* ... at most this many times */
  const double* hook_draws;        /* [n_hook_draws] uniform draws in [0, 1), consumed in order */
  int32_t n_hook_draws;
} pa_sched_config;

typedef struct pa_sched_plan_info {
  int32_t num_reqs;        /* requests scheduled in the pending plan */
  int32_t num_preempted;   /* preemptions done while planning it */
  int32_t num_copies;      /* copy-on-write block copies the step must run first */
  int64_t num_tokens;      /* sum of their query lengths */
  int32_t max_blocks;      /* longest block list among the scheduled requests */
  int32_t q_free, q_reserved, q_committed;   /* pool counters after planning */
} pa_sched_plan_info;

typedef struct pa_sched_metrics {
  /* pool state ([P5] "同时验证分配器与调度器") */
  int64_t q_free, q_reserved, q_committed, q_capacity;
  int64_t q_live;               /* distinct physical blocks referenced by requests */
  int64_t tail_waste;           /* sum over running requests of committed blocks * B - computed tokens */
  int64_t peak_used;            /* highest q_reserved + q_committed seen */
  int64_t allocation_failures;  /* free-block checks of running requests that failed (hook included) */
  /* scheduling */
  int64_t steps, rollbacks, admissions, preemptions, recompute_tokens, finished, cancelled;
  int64_t scheduled_tokens;     /* tokens of committed steps */
  int64_t running, waiting;
  /* reuse and reclaim */
  int64_t prefix_hit_tokens;    /* tokens attached from the prefix index */
  int64_t evictions;            /* cached blocks evicted under pressure */
  int64_t cow_copies;           /* copy-on-write block copies planned */
  int64_t cached_blocks;        /* blocks in the prefix index */
  int64_t evictable;            /* cached blocks no request references */
} pa_sched_metrics;

/* Create a scheduler.  Checks: positive sizes, block_order a permutation,
 * hook_prob in [0, 1], hook_max >= 0, n_hook_draws >= 0 (draws may be NULL
 * when 0).  *out receives the object (NULL on error). */
pa_status pa_sched_create(const pa_sched_config* cfg, pa_sched** out);
void pa_sched_destroy(pa_sched* s);

/* Queue a request at the back of the waiting queue.  request_id must be new;
 * prompt_len >= 1, output_len >= 1.  block_keys [n_keys] (may be NULL when
 * n_keys is 0, n_keys <= prompt_len / block_size): key j identifies the
 * content of the first (j+1)*block_size prompt tokens, including everything
 * that makes cached K/V reusable (token ids, model version, adapters, ...);
 * requests with keys share cached prefix blocks (see "Shared blocks"). */
pa_status pa_sched_add_request(pa_sched* s, int64_t request_id, int32_t prompt_len,
                               int32_t output_len, const uint64_t* block_keys, int32_t n_keys);

/* Parallel sampling: child_id (new) shares every block and the token state of
 * the RUNNING request parent_id and runs after every other running request;
 * output_len must exceed the tokens already generated.  PA_ERR_BAD_STATE if
 * a plan is pending or the parent is not running. */
pa_status pa_sched_fork(pa_sched* s, int64_t parent_id, int64_t child_id, int32_t output_len);

/* Plan one step (see the header comment); the plan stays pending until
 * commit or rollback.  info may be NULL. */
pa_status pa_sched_schedule(pa_sched* s, pa_sched_plan_info* info);

/* Copy the pending plan, in flattened order (request i of the step):
 *   request_ids [cap_reqs], num_computed [cap_reqs], query_lens [cap_reqs]
 *   block_table [cap_reqs, max_blocks_per_req] row-major, -1 padded: the
 *               request's blocks in logical order, covering
 *               num_computed + query_len positions
 *   preempted   [cap_preempted, 3] int64: (request id, tokens it held,
 *               blocks released), in the order they happened; may be NULL
 *               when cap_preempted is 0
 *   copies      [cap_copies, 2] int32: (source block, destination block) of
 *               each copy-on-write; may be NULL when cap_copies is 0
 * PA_ERR_BAD_SHAPE if a capacity is too small (nothing is written). */
pa_status pa_sched_plan_copy(const pa_sched* s, int64_t* request_ids, int32_t* num_computed,
                             int32_t* query_lens, int32_t cap_reqs, int32_t* block_table,
                             int32_t max_blocks_per_req, int64_t* preempted,
                             int32_t cap_preempted, int32_t* copies, int32_t cap_copies);

/* The step ran.  finished_ids [cap_finished] receives the requests that
 * finished (may be NULL when cap_finished is 0; PA_ERR_BAD_SHAPE and no
 * change if more finished than fit); *n_finished their count (may be NULL). */
pa_status pa_sched_commit(pa_sched* s, int64_t* finished_ids, int32_t cap_finished,
                          int32_t* n_finished);

/* The step failed: roll back the pending plan's reservations. */
pa_status pa_sched_rollback(pa_sched* s);

/* Cancel a request in any state (no-op if it already finished or was
 * cancelled); PA_ERR_OUT_OF_RANGE for an unknown id. */
pa_status pa_sched_cancel(pa_sched* s, int64_t request_id);

pa_status pa_sched_get_metrics(const pa_sched* s, pa_sched_metrics* m);

/* Detail of the last failing scheduler call on this thread ("" if none). */
const char* pa_sched_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_SCHED_H_ */
