/*
 * domino_bench.h — benchmark and test hooks of libdomino.so.
 *
 * These calls are outside the draft-head contract of domino.h.  They change
 * process-wide settings of the library (atomically, so reading them is
 * race-free, but a setting made on one thread applies to every thread's
 * later calls) and exist for measurement and for tests that compare the
 * chain's schedules.  A serving caller needs none of them.
 */
#ifndef DOMINO_BENCH_H
#define DOMINO_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "domino.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Timing hooks (hipEvent_t handles passed as void*).  While set, each later
 * domino_base_logits call records base_start on its stream right before its
 * GEMM launch and base_stop right after it; each domino_draft_chain call
 * records chain_start right before the launch(es) that run the P steps (after
 * the short prologue) and chain_stop right after them; each domino_tree_draft
 * call records the chain pair around all of its launches.  A NULL pair
 * disables that pair.  The events stay owned by the caller.
 */
void domino_set_timing_events(void *base_start, void *base_stop, void *chain_start, void *chain_stop);

/*
 * Chain scheduling.  0 (default): the library picks; one persistent launch
 * runs all P steps and, for bf16 weights where every workgroup's share fits,
 * keeps W2 on chip (registers and LDS) for all of them; otherwise the
 * stepwise schedule: per step a GRU launch, then the bottleneck and the W2
 * pass, in one launch for bf16 weights up to 16 sequences and in two
 * otherwise.  1: the stepwise schedule.  2: the persistent
 * launch with W2 read from memory every step.  3: the persistent launch,
 * keeping W2 on chip wherever its share fits (else as 2), whatever the batch.
 * All compute the same function with the same summation order, so their
 * outputs agree to the bit.  Returns the previous mode; any other value is
 * rejected with -1.
 */
int32_t domino_set_chain_mode(int32_t mode);

/*
 * Byte offset, inside a chain workspace for (dims, batch), of P + 1 uint64
 * timestamps of the device's constant 100 MHz clock that the one-launch
 * schedule writes: entry p (p < P) when step p starts in the first
 * workgroup, entry P when that workgroup finishes.  Three-launch schedules
 * leave them untouched.  Returns 0 for arguments domino_workspace_size
 * rejects.
 */
size_t domino_chain_stamp_offset(const domino_dims *dims, int32_t batch);

#ifdef __cplusplus
}
#endif

#endif /* DOMINO_BENCH_H */
