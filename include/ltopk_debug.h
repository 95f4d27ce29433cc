/*
 * ltopk_debug.h -- test hooks of libltopk.so (not for production callers).
 *
 * These change process-wide state (atomic integers) that later calls of
 * lt_topk_run and lt_topk_blocks read when they choose their launches; a call
 * running concurrently with a change sees either the old or the new setting.
 */
#ifndef LTOPK_DEBUG_H
#define LTOPK_DEBUG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Kernel choice for rows without a candidate list: 0 = automatic (default),
 * 1 = always split rows over workgroups (launched in as many row groups as
 * fit on the device at once), 2 = always one streaming workgroup per row,
 * 3 = one 1024-thread workgroup per whole row when n_max <= 32768, and per
 * candidate list of up to 2048 blocks of eight (else the automatic choice).
 * Any other value is ignored. Returns the previous setting.
 */
int lt_debug_force_path(int path);

/*
 * 1: rows split over several workgroups always take the exact fallback in
 * their last workgroup (re-read the row, select digit by digit) instead of
 * the gathered candidates; 0: normal operation (default). Returns the
 * previous setting.
 */
int lt_debug_force_fallback(int on);

/*
 * Threshold mode of plain rows split over 2 to 64 workgroups (k <= 1024):
 * 0 = the mode word in the row's workspace record decides (default; see
 * lt_topk_run), 1 = never sample (each workgroup bounds its candidates by its
 * own scores), 2 = always take the threshold from the row's sample. Any other
 * value is ignored. Returns the previous setting.
 */
int lt_debug_force_sample(int mode);

/*
 * Shape of the (first) launch lt_topk_run makes for B rows of n_max scores
 * without a candidate list and k <= 512: grid and block size. Returns 0 for the split
 * kernel, 1 for the streaming kernel, 2 for the whole-row kernel, -1 on bad
 * arguments or when the device cannot be queried. Host only; launches
 * nothing.
 */
int lt_debug_launch_shape(int32_t B, int32_t n_max, int32_t *grid_x, int32_t *grid_y,
                          int32_t *block);

/*
 * Launch an empty kernel with the given grid and block size on `stream`
 * (a hipStream_t; NULL = null stream). Used to measure the launch floor that
 * latency-bound calls are compared against. Returns 0, or -1 on a bad shape
 * or a launch error.
 */
int lt_debug_empty_launch(int32_t grid_x, int32_t grid_y, int32_t block, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LTOPK_DEBUG_H */
