/*
 * ltopk_debug.h -- test hooks of libltopk.so (not for production callers).
 *
 * These change process-wide state read by later calls of lt_topk_run and
 * lt_topk_blocks; set them only while no call is in flight.
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
 * fit on the device at once), 2 = always one streaming workgroup per row.
 * Any other value is ignored. Returns the previous setting.
 */
int lt_debug_force_path(int path);

/*
 * Bound on the polls a workgroup makes while waiting at the per-row barrier
 * of the split kernel (default 1 << 24, about half a second). When it runs
 * out the workgroup sets bit 0 of the row's status word in the workspace and
 * carries on, so the kernel always finishes; that call's output is then
 * undefined and the workspace must be zero-filled again before reuse.
 * Returns the previous bound.
 */
uint32_t lt_debug_set_spin_limit(uint32_t polls);

/*
 * Byte offset of row r's status word inside a workspace (0 on success; bit 0
 * set when a barrier wait ran out). Pure host arithmetic.
 */
size_t lt_debug_status_offset(int32_t row);

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
