/*
 * pkv_sched.h -- host block manager and continuous-batching scheduler that
 * sits directly above the paged KV kernels of pkv.h.
 *
 * Defined by "Build a Mini vLLM: Paged KV Cache and Continuous Batching From
 * Scratch" ([MV]):
 *   section 2 "The paged KV cache": the BlockManager -- a free list of every
 *     block id (a new block is taken from the end of the list, released
 *     blocks are appended in table order), per-sequence tables and lengths, a
 *     new block when a sequence's length reaches a multiple of the block size,
 *     admission only when ceil((prompt + 1) / block_size) blocks are free;
 *   section 5 "The engine": requests wait in FIFO order; each step admits (and
 *     prefills) requests up to max_batch while blocks last -- every step in
 *     continuous mode, only when nothing runs in static mode -- then, while the
 *     running requests whose length is a multiple of the block size outnumber
 *     the free blocks, evicts the youngest running request (recompute
 *     preemption: its blocks are freed, the tokens it generated are appended to
 *     its prompt and it goes back to the front of the queue), then decodes one
 *     token for every running request (writing the previous token's K/V), and
 *     retires requests that reached their stop length;
 *   section 6 "Memory: reserved vs allocated vs used": per-step accounting;
 *   section 8 "Preemption: when the pool runs dry".
 *
 * The scheduler only decides; it never touches device memory. Each
 * pkv_sched_step() returns the rows to prefill (positions 0 .. len-1 of the
 * admitted requests) and the rows to decode (one new token per running
 * request at position pos, attending 0 .. pos), with their block tables, for
 * the caller to run through pkv_slot_mapping / pkv_write / pkv_prefill /
 * pkv_decode_step. All pointers are host pointers owned by the caller.
 * Not thread-safe: one scheduler per thread.
 */
#ifndef PKV_SCHED_H
#define PKV_SCHED_H

#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_sched pkv_sched;

/* One step's work. The caller provides the arrays: *_rid and *_len / *_pos
 * hold max_batch entries, *_tables max_batch * max_blocks_per_seq entries
 * (row-major; entries past a row's blocks are 0). */
typedef struct pkv_sched_step_out {
  int32_t num_prefill;    /* requests admitted this step and still running     */
  int32_t num_decode;     /* running requests, each decoded one token          */
  int32_t num_preempted;  /* evictions this step                               */
  int32_t num_finished;   /* requests retired this step                        */
  int32_t* prefill_rid;
  int32_t* prefill_len;   /* prompt tokens written at positions 0 .. len-1     */
  int32_t* prefill_tables;
  int32_t* decode_rid;
  int32_t* decode_pos;    /* position of the token written and attended from   */
  int32_t* decode_tables;
} pkv_sched_step_out;

typedef struct pkv_sched_stats {
  int64_t steps;              /* steps that decoded (history entries)            */
  int64_t preemptions;
  int64_t tokens_generated;   /* over retired requests                           */
  int64_t requests_done;
  int64_t sum_running;        /* sums over steps, after retirement:              */
  int64_t sum_naive_tokens;   /*   prompt + max_new of each running request      */
  int64_t sum_allocated_tokens; /* blocks in use * block_size                    */
  int64_t sum_used_tokens;    /*   tokens held                                   */
} pkv_sched_stats;

/* NULL on bad sizes (num_blocks, block_size, max_batch, max_blocks_per_seq
 * must be >= 1). continuous: 1 = refill every step, 0 = static batches. */
pkv_sched* pkv_sched_create(int32_t num_blocks, int32_t block_size, int32_t max_batch,
                            int32_t continuous, int32_t max_blocks_per_seq);
void pkv_sched_destroy(pkv_sched* s);

/* Queue a request (FIFO). prompt_len >= 1, max_new >= 1, 1 <= stop_after;
 * rid must be unique. PKV_ERR_CAPACITY if its prompt plus stop length can
 * never fit max_blocks_per_seq blocks. */
pkv_status pkv_sched_submit(pkv_sched* s, int32_t rid, int32_t prompt_len, int32_t max_new,
                            int32_t stop_after);

/* Requests waiting or running. */
int32_t pkv_sched_pending(const pkv_sched* s);

/* One engine step. PKV_ERR_NULL if s, out or one of out's arrays is NULL
 * (nothing changes then); PKV_ERR_CAPACITY if nothing can run and nothing
 * fits (a request larger than the whole pool). */
pkv_status pkv_sched_step(pkv_sched* s, pkv_sched_step_out* out);

pkv_status pkv_sched_get_stats(const pkv_sched* s, pkv_sched_stats* st);

/* Per-step history (running requests, naive, allocated and used tokens),
 * first min(cap, steps) entries; returns the number written. */
int64_t pkv_sched_history(const pkv_sched* s, int32_t* running, int64_t* naive,
                          int64_t* allocated, int64_t* used, int64_t cap);

#ifdef __cplusplus
}
#endif

#endif /* PKV_SCHED_H */
