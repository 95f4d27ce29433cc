/*
 * ltopk.h -- top-k index selection for compressed sparse attention (CSA) on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation. DeepSeek-V4's CSA layer compresses the KV cache 4:1 and lets
 * each query attend only to the compressed positions its indexer scores
 * highest (AICon 2026 Shenzhen speaker page, aicon.infoq.cn: abstract and
 * outline 一.1; a CSA position is the token position divided by 4, outline
 * 二.1). Each index-source layer keeps at most 512 of them; one layer instead
 * picks at most 2048 blocks of eight positions, and later layers restrict their
 * top-512 to those blocks ("SGLang 与 Miles 为 DeepSeek-V4.1 提供首日支持",
 * xhh.club: Q&A on cross-layer sharing). The top-k step is the one the talk
 * notes on devpress.csdn.net (section 3.2, LightningTopK) time at a 1M-token
 * context and batch size 1.
 *
 * Selection rule (the pages fix k and "at most"; the rest is the reading
 * taken). For row r with valid length len (clamped to [0, n_max]) the valid
 * positions are V = {i : 0 <= i < len} (intersected with the candidate
 * positions when a candidate list is given). Positions are ordered by score,
 * highest first, in the real-number order with -0.0 == +0.0, +inf highest,
 * -inf the lowest non-NaN value and every NaN below -inf; equal scores order
 * by lower index first. The result is the first m = min(k, |V|) positions in
 * that order. Exactly one index set satisfies this, so results are
 * reproducible bit for bit.
 *
 * Conventions for every call:
 *   - host functions; every pointer argument is DEVICE memory unless stated;
 *   - asynchronous on `stream` (0 = the null stream); no call synchronises,
 *     allocates device memory or throws;
 *   - output slots [0, m) of a row hold the selected indices in no particular
 *     order; slots [m, k) hold -1;
 *   - the caller owns every buffer.
 *
 * Workspace. When a row is split over several workgroups, they publish
 * candidates and count themselves done in a caller-provided workspace. It
 * must be zero-filled once before its first use; every call returns its
 * counters to zero (the other bytes are scratch), so no clearing is needed
 * between calls and calls can be captured in a graph as they are. Calls that
 * may run concurrently (different streams) need distinct workspaces. Query
 * the size with lt_topk_workspace_bytes; a size of 0 means no workspace is
 * used and `workspace` may be NULL.
 *
 * The workspace also carries one mode word per row record from a call to the
 * next (rows of plain scores split over 2 to 64 workgroups, k <= 1024): which
 * of two exact ways of bounding the workgroups' candidates the next call on
 * that row record uses. A row whose best scores cluster in a few chunks
 * switches the next call to a threshold taken from a sample of the row; a
 * row whose best scores are spread switches it back. The selected indices
 * never depend on the mode, only the time does: a call on a clustered row
 * after a call on a spread one (or on a fresh workspace) takes a second pass
 * over the clustered chunks.
 */
#ifndef LTOPK_H
#define LTOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same object as hipStream_t; declared here so the header needs no HIP. */
typedef struct ihipStream_t *lt_stream_t;

typedef enum {
    LT_OK = 0,
    LT_EINVAL = 1, /* invalid argument; nothing was launched                 */
    LT_ENOSPC = 2, /* workspace smaller than lt_topk_workspace_bytes(...)    */
    LT_EHIP = 3    /* the HIP runtime reported an error at launch            */
} lt_status;

/* Largest supported k (and kb). */
#define LT_K_MAX 4096

/* Longest virtual rows of the forms that only the split kernel takes (1024
 * workgroups per row): blocks per row for a block stage with block_size != 8,
 * and candidate slots per row for lists with block_size != 8. */
#define LT_MAX_SPLIT_BLOCKS 4194304
#define LT_MAX_SPLIT_SLOTS 8388608

/*
 * Optional candidate restriction, in block form (the shared-candidate layers
 * on the V4.1 page, Q&A on cross-layer sharing).
 *   blocks     : device int32 [B, n_blocks], row-major. Block id b stands for
 *                positions [b*block_size, b*block_size + block_size). Ids < 0
 *                mark empty slots; ids whose positions all lie at or beyond
 *                the row's length contribute nothing. A row must not list the
 *                same id twice (the block stage never does); if it does, the
 *                result is unspecified.
 *   n_blocks   : >= 1 (2048 in the shared-candidate layers)
 *   block_size : >= 1 (8 in the shared-candidate layers)
 */
typedef struct {
    const int32_t *blocks;
    int32_t n_blocks;
    int32_t block_size;
} lt_cand_t;

/*
 * Bytes of workspace lt_topk_run / lt_topk_blocks need for a batch of B rows
 * of n_max scores. For the candidate form pass n_max = max(n_max,
 * n_blocks * block_size). Pure host arithmetic; never touches the GPU.
 * Returns 0 when no workspace is needed.
 */
size_t lt_topk_workspace_bytes(int32_t B, int32_t n_max, int32_t k);

/*
 * Top-k positions per row.
 *   scores     : device fp32 [B rows, row_stride], 16-byte aligned; row r
 *                starts at scores + r*row_stride; row_stride % 4 == 0 and
 *                row_stride >= n_max. Rows must be readable up to n_max
 *                rounded up to a multiple of 4 (the buffer holds at least
 *                (B-1)*row_stride + round_up(n_max, 4) floats). Positions at
 *                or beyond a row's length are never used (any bytes, NaN and
 *                +inf included, are ignored there).
 *   lengths    : device int32 [B]; valid length per row, clamped to [0, n_max]
 *   B          : rows, >= 0 (0 is a no-op)
 *   n_max      : positions per row, >= 0
 *   k          : 1 <= k <= LT_K_MAX
 *   cand       : host pointer to a candidate restriction, or NULL for none;
 *                the struct is read during the call, its `blocks` array on the
 *                device
 *   out_idx    : device int32 [B, k], row-major
 *   workspace  : device buffer of ws_bytes (see above)
 *   stream     : HIP stream the work is enqueued on
 * Returns LT_EINVAL without launching for: NULL scores/lengths/out_idx,
 * B < 0, n_max < 0, k outside [1, LT_K_MAX], row_stride < n_max or
 * row_stride % 4 != 0, scores not 16-byte aligned, workspace not 16-byte
 * aligned, a candidate struct with NULL blocks, n_blocks < 1 or
 * block_size < 1, and a candidate list longer than LT_MAX_SPLIT_SLOTS slots
 * (n_blocks * block_size) unless block_size == 8 and n_max <= 536,866,816
 * (such lists are selected by workgroups that split the list, at most 1024 of
 * them). LT_ENOSPC if ws_bytes is below what this batch needs (or workspace
 * is NULL while bytes are needed); nothing is launched and out_idx is left
 * untouched. LT_EHIP if a launch failed.
 */
lt_status lt_topk_run(const float *scores, int64_t row_stride, const int32_t *lengths,
                      int32_t B, int32_t n_max, int32_t k, const lt_cand_t *cand,
                      int32_t *out_idx, void *workspace, size_t ws_bytes,
                      lt_stream_t stream);

/*
 * lt_topk_run without a workspace argument, for callers that cannot allocate
 * device memory: code under stream/graph capture, serving loops and
 * harnesses that forbid allocation. Same arguments (less workspace and
 * ws_bytes), same results, same kernels.
 *
 * Rows split over several workgroups exchange candidates through a buffer
 * built into the library instead: LT_NOALLOC_BYTES (5,193,728 bytes, the
 * records of LT_NOALLOC_SPLIT_ROWS = 64 split rows) of device memory per GPU,
 * held from the first call on that GPU until the process ends. A call whose
 * split launch needs more records (more than 64 rows that each span several
 * workgroups, e.g. a batch of 65 rows of 262,144 scores) returns LT_ENOSPC
 * without launching anything; batches that one workgroup per row serves
 * (short rows, or many long rows streamed one wavefront each) have no limit.
 * Nothing is allocated: no hipMalloc, hipFree or allocating library routine.
 *
 * Every call on one GPU shares that GPU's buffer. Calls that may overlap in
 * time on one GPU (different streams without an ordering between them, or
 * several host threads) race and give undefined results; the caller orders
 * them. The buffer's counters are cleared by a small kernel enqueued before
 * the first split launch on each GPU (and, under stream capture, recorded
 * into the graph), after which every call leaves them at zero.
 */
#define LT_NOALLOC_SPLIT_ROWS 64
#define LT_NOALLOC_BYTES 5193728
lt_status lt_topk_run_noalloc(const float *scores, int64_t row_stride, const int32_t *lengths,
                              int32_t B, int32_t n_max, int32_t k, const lt_cand_t *cand,
                              int32_t *out_idx, lt_stream_t stream);

/*
 * Block stage of the shared-candidate layers (V4.1 page, Q&A on cross-layer
 * sharing): the row's positions are grouped into blocks of block_size
 * (block b = positions [b*block_size, (b+1)*block_size)); the blocks holding at
 * least one valid position (b < ceil(len / block_size)) are scored by the
 * highest score among their valid positions (NaN lowest; how a block is scored
 * is the reading taken, the pages do not say), and the top-kb block ids are
 * returned by the selection rule above, block ids acting as indices.
 *   out_blocks : device int32 [B, kb]; slots [0, min(kb, nb)) hold block ids in
 *                no particular order, the rest -1.
 * Arguments and errors as lt_topk_run, with block_size >= 1 and
 * 1 <= kb <= LT_K_MAX; LT_EINVAL also when block_size != 8 and the row has
 * more than LT_MAX_SPLIT_BLOCKS blocks (ceil(n_max / block_size)). Pass
 * out_blocks to lt_topk_run as lt_cand_t.blocks (n_blocks = kb) to run the
 * restricted top-k.
 */
lt_status lt_topk_blocks(const float *scores, int64_t row_stride, const int32_t *lengths,
                         int32_t B, int32_t n_max, int32_t block_size, int32_t kb,
                         int32_t *out_blocks, void *workspace, size_t ws_bytes,
                         lt_stream_t stream);

/*
 * Both stages of a shared-candidate layer (V4.1 page, Q&A on cross-layer
 * sharing): the top-kb blocks of each row, as lt_topk_blocks writes them to
 * out_blocks, and the row's top-k positions inside those blocks, as
 * lt_topk_run with lt_cand_t{out_blocks, kb, block_size} writes them to
 * out_idx: those two calls, stream-ordered on one workspace.
 *   out_blocks : device int32 [B, kb]   out_idx : device int32 [B, k]
 * Arguments, workspace (lt_topk_workspace_bytes(B, n_max, k) covers both
 * stages) and errors as the two calls; LT_EINVAL also for a NULL out_idx or k
 * outside [1, LT_K_MAX].
 */
lt_status lt_topk_two_stage(const float *scores, int64_t row_stride, const int32_t *lengths,
                            int32_t B, int32_t n_max, int32_t block_size, int32_t kb, int32_t k,
                            int32_t *out_blocks, int32_t *out_idx, void *workspace,
                            size_t ws_bytes, lt_stream_t stream);

/*
 * Output variants for the consumer of a selection: CSA's sparse attention over
 * the selected compressed positions (AICon 2026 Shenzhen speaker page,
 * aicon.infoq.cn: abstract and outline 一.1). The pages give no layout for what
 * the consumer receives; these take the plainest reading (indices in a fixed
 * order, the scores at them, the selected cache rows themselves). In both
 * calls a slot holding an index outside [0, n) (n = n_max, resp. n_kv) counts
 * as empty, like a -1 slot.
 */
typedef enum {
    LT_ORDER_ASIS = 0,  /* slots left as they are (values only)                   */
    LT_ORDER_INDEX = 1, /* ascending index, then the empty slots as -1            */
    LT_ORDER_RANK = 2   /* selection order: higher score first, lower index first
                           among equal scores, -0.0 == +0.0, NaN below -inf; then
                           the empty slots as -1                                   */
} lt_order;

/*
 * Reorder each row's slots in place and/or return the score at each slot.
 *   scores   : as for lt_topk_run (device fp32 [B, row_stride], positions
 *              [0, n_max) readable); may be NULL if order != LT_ORDER_RANK and
 *              out_vals == NULL
 *   B, n_max : rows; positions per row
 *   k        : slots per row, 1 <= k <= LT_K_MAX
 *   order    : an lt_order value
 *   idx      : device int32 [B, k], row-major, e.g. lt_topk_run's out_idx;
 *              rewritten in place (unchanged with LT_ORDER_ASIS). Repeated
 *              indices are kept.
 *   out_vals : device fp32 [B, k] or NULL; receives scores[r, idx[r, j]] after
 *              the reordering (the score's exact bits), -inf for empty slots
 * Returns LT_EINVAL without launching for: NULL idx, B < 0, n_max < 0, k
 * outside [1, LT_K_MAX], an unknown order, or (when scores are needed) NULL
 * scores or row_stride < n_max. LT_EHIP if a launch failed. B == 0, or
 * LT_ORDER_ASIS with out_vals == NULL, launches nothing.
 */
lt_status lt_topk_order(const float *scores, int64_t row_stride, int32_t B, int32_t n_max,
                        int32_t k, int32_t order, int32_t *idx, float *out_vals,
                        lt_stream_t stream);

/*
 * Gather the compressed-KV cache rows a selection names:
 *   out[r, j, :] = kv[r * kv_batch_stride + idx[r, j] * kv_stride, + row_bytes)
 * with zero bytes for empty slots.
 *   kv              : device, 16-byte aligned; one cache of n_kv rows per
 *                     batch row (kv_batch_stride bytes apart), or one cache
 *                     shared by every row (kv_batch_stride = 0)
 *   kv_stride       : bytes between cache rows, >= row_bytes, % 16 == 0
 *   kv_batch_stride : >= 0, % 16 == 0
 *   n_kv            : rows per cache, >= 0
 *   row_bytes       : bytes copied per slot, 16 <= row_bytes <= 1 MiB,
 *                     % 16 == 0
 *   idx             : device int32 [B, k] (any order; ascending index reads
 *                     the cache in address order)
 *   out             : device [B, k, row_bytes], 16-byte aligned
 * Returns LT_EINVAL without launching for: NULL kv/idx/out, B < 0, k outside
 * [1, LT_K_MAX], n_kv < 0, a row_bytes, kv_stride or kv_batch_stride outside
 * the limits above, kv or out not 16-byte aligned. LT_EHIP if a launch failed.
 */
lt_status lt_gather_rows(const void *kv, int64_t kv_stride, int64_t kv_batch_stride, int64_t n_kv,
                         int32_t row_bytes, const int32_t *idx, int32_t B, int32_t k, void *out,
                         lt_stream_t stream);

/* Static, human-readable name of a status code. Never NULL. */
const char *lt_status_str(lt_status status);

#ifdef __cplusplus
}
#endif

#endif /* LTOPK_H */
