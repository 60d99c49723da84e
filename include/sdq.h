/*
 * sdq.h -- C ABI of libsdq.so: one long-context decode step of sparse
 * attention on an MI355X (gfx950).
 *
 * The step: score every cached key through a cheap index, keep the top-k per
 * KV head, read those bf16 K/V rows by index and run renormalised softmax
 * attention over them.  Three index formats are supported:
 *   - per-channel 4-bit bit planes read under a per-query plan (Fathom
 *     summary page: bit-plane and reverse water-filling paragraphs),
 *   - 32-bit signatures scored by XOR/popcount (HashAttention study notes,
 *     sec. 2.2),
 *   - per-block min/max key summaries (OasisKV review, Quest-style block
 *     summaries in the background and core-method sections).
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers owned by the caller, unless a comment says
 *     host.  The library never allocates or frees; scratch memory is a
 *     caller-supplied workspace whose size the matching *_workspace_bytes()
 *     returns.
 *   - Every call is asynchronous on the caller's stream (0 = the null
 *     stream).  Results are valid once the stream reaches that point.
 *   - Every call validates its arguments before launching anything; a call
 *     that returns an error has launched nothing.  Return values:
 *       SDQ_OK (0), SDQ_EINVAL (-1: null pointer, bad size or shape),
 *       SDQ_ENOTSUP (-2), SDQ_EHIP (-3: a HIP launch/runtime error).
 *     sdq_last_error() returns a message for the calling thread's last error.
 *   - The library holds no global mutable state apart from that per-thread
 *     message and the static per-GPU scratch of topk_select_noalloc; calls
 *     on different streams may run concurrently if their output and
 *     workspace buffers do not overlap (topk_select_noalloc calls on one GPU
 *     share their scratch and must not overlap).
 *   - Head dimension d must be 128 in this version.
 *   - bf16 and fp16 data are passed as uint16_t bit patterns.
 */
#ifndef SDQ_H
#define SDQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDQ_OK 0
#define SDQ_EINVAL (-1)
#define SDQ_ENOTSUP (-2)
#define SDQ_EHIP (-3)

/* 64-token blocks per group maximum (fathom_scan's group_max): 512 tokens */
#define SDQ_GROUP_BLOCKS 8

/* key kinds for topk_select */
#define SDQ_KEY_F32_MAX 0 /* float32 scores, largest first        */
#define SDQ_KEY_U8_MIN 1  /* uint8 distances, smallest first      */

/* Message describing the calling thread's most recent error ("" if none). */
const char* sdq_last_error(void);

/* ABI version of this header (incremented on incompatible changes).
 * Version 2: row capacities (n_cap, nb_cap) on every call that reads
 * per-token cache arrays; fathom_append, minmax_append, oasis_select and
 * oasis_fetch.
 * Version 3: group maxima (SDQ_GROUP_BLOCKS blocks of 64 tokens) written by
 * fathom_scan and fathom_plan_scan and read by topk_select_block_max_split. */
int sdq_abi_version(void);

/* ------------------------------------------------------------------------
 * Index construction (the step before the decode path)
 * --------------------------------------------------------------------- */

/* fathom_ingest -- build the bit-plane index of a bf16 key cache.
 * Fathom summary, bit-plane paragraph: keys are quantised per channel to
 * 4-bit uniform codes with one fp16 scale per 64-token block, and each code
 * bit is stored as its own channel-major plane.
 *   keys    bf16 [G][n][d]   key cache, token-major rows
 *   planes  uint32 [G][d][4][n/32]  out.  Plane p holds code bit (3-p), so
 *           plane 0 is the MSB and a channel's first t planes form one
 *           contiguous range of t*n/8 bytes.  Token i is bit (i & 31) of
 *           word (i >> 5).
 *   meta    uint32 [G][d][n/64]  out.  Low half: fp16 scale; high half:
 *           fp16 offset of that channel's 64-token block.
 * Quantiser (float32): offset = fp16(min), scale = fp16((max-min)/15),
 * code = clamp(rint((x - offset)/scale), 0, 15), code 0 where scale is 0.
 * Keys must be finite and within fp16 range; the key pointer must be 16-byte
 * aligned.
 * Errors: SDQ_EINVAL if a pointer is null or keys misaligned, G < 1, n < 64,
 * n % 64 != 0 or d != 128. */
int fathom_ingest(const uint16_t* keys, int G, int n, int d, uint32_t* planes, uint32_t* meta,
                  hipStream_t stream);

/* fathom_append -- add a decode step's new keys to a growing bit-plane index
 * (Fathom summary, bit-plane paragraph; the per-step compressed-key update
 * of the OasisKV review).  The cache has a fixed row capacity of n_cap
 * tokens and holds its first n_old + n_new; the call quantises every 64-token
 * block that holds one of the tokens [n_old, n_old + n_new).  A block whose
 * tokens are not all present yet (the open block) is quantised over the
 * tokens it holds, with its own scale and offset, and its absent tokens get
 * code 0; it is quantised again by later appends until it is full, and is
 * then identical to what fathom_ingest gives for the same 64 keys.
 *   keys    bf16 [G][n_cap][d]   key cache, tokens [0, n_old + n_new) valid
 *   planes  uint32 [G][d][4][n_cap/32]  in/out, the fathom_ingest layout with
 *           rows n_cap tokens long; blocks before n_old/64 and after the
 *           last touched block are left as they are.
 *   meta    uint32 [G][d][n_cap/64]  in/out, likewise.
 * n_new == 0 is a no-op.
 * Errors: SDQ_EINVAL on null pointers, keys not 16-byte aligned, G < 1,
 * d != 128, n_cap not a positive multiple of 64 below 2^25, n_old < 0,
 * n_new < 0, n_old + n_new > n_cap. */
int fathom_append(const uint16_t* keys, int G, int d, int n_cap, int n_old, int n_new,
                  uint32_t* planes, uint32_t* meta, hipStream_t stream);

/* minmax_summarize -- per-block min/max key summaries (OasisKV review,
 * Quest-style summaries: one minimum and one maximum vector per logical
 * block, per dimension).
 *   keys  bf16 [RG][n][d];   bmin, bmax  fp16 [RG][n/block][d]  out.
 * The block minimum is rounded to fp16 downwards and the maximum upwards, so
 * each summary still bounds every key of its block.
 * Errors: SDQ_EINVAL on null pointers, RG < 1, block < 1, n % block != 0,
 * d != 128. */
int minmax_summarize(const uint16_t* keys, int RG, int n, int d, int block, uint16_t* bmin,
                     uint16_t* bmax, hipStream_t stream);

/* minmax_append -- add new keys to growing min/max summaries (OasisKV
 * review: summaries are updated as the cache grows).  Rows hold n_cap tokens,
 * the first n_old + n_new present; every block holding one of the tokens
 * [n_old, n_old + n_new) is summarised again over its present tokens (a
 * partly filled last block bounds exactly the keys it holds).
 *   keys  bf16 [RG][n_cap][d];  bmin, bmax  fp16 [RG][n_cap/block][d] in/out
 * n_new == 0 is a no-op.
 * Errors: SDQ_EINVAL on null pointers, RG < 1, d != 128, block < 1, n_cap not
 * a positive multiple of block, n_old < 0, n_new < 0, n_old + n_new > n_cap. */
int minmax_append(const uint16_t* keys, int RG, int d, int n_cap, int n_old, int n_new, int block,
                  uint16_t* bmin, uint16_t* bmax, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode step
 * --------------------------------------------------------------------- */

/* fathom_plan -- per-query read plan by reverse water-filling.
 * Fathom summary, water-filling paragraph: channel j contributes
 * q_j^2 * var_j to the score variance, each extra bit cuts the remaining
 * error of that channel by 4, and budget_bits plane bits are spread over the
 * channels (0..4 each) by this marginal gain; query heads under one KV head
 * share one plan.
 *   q        float32 [G*H_grp][d]  query rows; rows g*H_grp..g*H_grp+H_grp-1
 *            belong to KV head g
 *   key_var  float32 [G][d]        calibrated key variance per channel (>= 0;
 *            a weight that comes out negative or NaN is read as zero gain)
 *   depth    uint8 [G][d]   out: bits to read per channel (0..4)
 *   qbar     float32 [G][d] out: the group's query sum, added in head order
 * Exactly min(budget_bits, 4d) bits are given out per KV head: the items
 * w_j * 4^-t (w_j = (qbar_j*qbar_j)*var_j, float32) are taken in the order
 * (gain desc, channel asc, bit asc).
 * Errors: SDQ_EINVAL on null pointers, G < 1, H_grp < 1, d != 128,
 * budget_bits < 0. */
int fathom_plan(const float* q, const float* key_var, int G, int H_grp, int d, int budget_bits,
                uint8_t* depth, float* qbar, hipStream_t stream);

/* fathom_plan_uniform -- the uniform-depth baseline plan the Fathom summary
 * compares against (a fixed set of channels read at full depth): the
 * n_channels channels of largest (qbar_j*qbar_j)*var_j, ties to the lower
 * channel, each at depth 4.  Same arguments and errors as fathom_plan with
 * 0 <= n_channels <= d in place of the budget. */
int fathom_plan_uniform(const float* q, const float* key_var, int G, int H_grp, int d,
                        int n_channels, uint8_t* depth, float* qbar, hipStream_t stream);

/* fathom_gather -- copy the active channels' plane prefixes from host memory
 * into HBM (Fathom summary, offload paragraph: host planes are contiguous
 * per channel and one gather moves the active prefixes over PCIe before the
 * scan).
 *   planes_host, meta_host  HOST pointers to pinned, device-mapped memory
 *           (hipHostMalloc) in the fathom_ingest layout
 *   depth   uint8 [G][d] device, a plan from fathom_plan*
 *   planes_dev, meta_dev  device buffers in the same layout; for every
 *           channel with depth t > 0 the first t planes and the meta row are
 *           written, everything else is left untouched.
 * Run it on a side stream ordered after the plan with events.
 * Both layouts have rows of n_cap tokens (fathom_append); the words of the
 * first n tokens, n rounded up to 64, are copied.
 * Errors: SDQ_EINVAL on null pointers, bad sizes (as fathom_scan), or host
 * memory the device cannot address. */
int fathom_gather(const uint32_t* planes_host, const uint32_t* meta_host, const uint8_t* depth,
                  int G, int d, int n, int n_cap, uint32_t* planes_dev, uint32_t* meta_dev,
                  hipStream_t stream);

/* fathom_scan -- approximate scores from the plane prefixes.
 * For every KV head g and token i:
 *   s[g][i] = sum over channels j with t_j = depth[g][j] > 0 of
 *             qbar[g][j] * (offset + scale * (c * 2^(4-t_j) + (2^(4-t_j)-1)/2))
 * where c is the t_j-bit code read from the first t_j planes and scale/offset
 * are that channel's 64-token block metadata (the midpoint of the t-bit bin,
 * the 4-bit dequantisation at t = 4).  Unread channels contribute nothing and
 * their metadata is not read; depths outside 1..4 count as unread.
 * Accumulation is float32 (each channel's code times its weight is added with
 * one fused multiply-add).
 *   planes, meta  as fathom_append: rows of n_cap tokens (n_cap = n for an
 *                 index built by fathom_ingest); the first n tokens are
 *                 scored, n any value in [1, n_cap]
 *   depth, qbar   as fathom_plan
 *   scores        float32 [G][n64] out, n64 = n rounded up to a multiple of
 *                 64, 16-byte aligned; tokens [n, n64) (the absent part of
 *                 an open block) are written as -inf
 *   block_max     float32 [G][n64/64] out, or NULL: the maximum score of
 *                 every 64-token block (input of topk_select_block_max)
 *   group_max     float32 [G][ceil(n64/64 / SDQ_GROUP_BLOCKS)] out, or NULL:
 *                 the maximum score of every group of SDQ_GROUP_BLOCKS
 *                 blocks (the last group may be shorter); input of
 *                 topk_select_block_max_split
 * Errors: SDQ_EINVAL on null pointers, G < 1, n_cap not a positive multiple
 * of 64, n outside [1, n_cap], n_cap >= 2^25 (one head's planes are addressed
 * with 31-bit offsets), d != 128, misaligned scores. */
int fathom_scan(const uint32_t* planes, const uint32_t* meta, const uint8_t* depth,
                const float* qbar, int G, int d, int n, int n_cap, float* scores,
                float* block_max, float* group_max, hipStream_t stream);

/* fathom_plan_scan -- fathom_plan (uniform == 0) or fathom_plan_uniform
 * (uniform != 0) followed by fathom_scan, in one launch (Fathom summary,
 * water-filling and bit-plane paragraphs: the plan is per query, the scan
 * reads what the plan selects).  Every scan workgroup derives its KV head's
 * plan with the same computation as fathom_plan, so plan and scores are
 * identical to the two separate calls; this removes one launch and one
 * dependent memory round trip from the decode step.
 *   q, key_var, H_grp      as fathom_plan
 *   budget                 budget_bits, or n_channels when uniform != 0
 *   planes, meta, G, d, n, n_cap  as fathom_scan
 *   depth, qbar            out, or both NULL: the plan, as fathom_plan writes it
 *   scores, block_max, group_max  as fathom_scan
 * Errors: the union of fathom_plan's and fathom_scan's, and SDQ_EINVAL when
 * exactly one of depth and qbar is NULL. */
int fathom_plan_scan(const float* q, const float* key_var, int H_grp, int budget, int uniform,
                     const uint32_t* planes, const uint32_t* meta, int G, int d, int n,
                     int n_cap, uint8_t* depth, float* qbar, float* scores, float* block_max,
                     float* group_max, hipStream_t stream);

/* topk_select -- per-row top-k (HashAttention study notes, sec. 2.1 TOPK and
 * sec. 3.1 fixed positions; OasisKV review, per-KV-head top-K).
 *   keys      [rows][n]: float32 (SDQ_KEY_F32_MAX, largest first; not NaN,
 *             -inf allowed (fathom_scan's pad value), -0 equals +0) or uint8
 *             (SDQ_KEY_U8_MIN, smallest first)
 *   idx_out   int32 [rows][k + n_sink + n_local] out
 * Per row: positions [0, n_sink) and [n - n_local, n) are always kept and do
 * not compete; the k best of [n_sink, n - n_local) are added, equal keys
 * going to the lower index.  Indices are written in ascending order.  When k
 * is at least n - n_sink - n_local every index 0..n-1 is written and the
 * rest of the row is filled with -1.
 *   ws, ws_bytes  workspace of at least topk_select_workspace_bytes() bytes
 *             (float32 rows: per-row histograms and candidate lists; uint8
 *             rows of 32768 keys or more: one 256-entry histogram per 16384
 *             keys per row; a few bytes otherwise).  Its contents on entry do
 *             not matter and calls on one workspace must not overlap.
 * Errors: SDQ_EINVAL on null pointers, rows < 1, n < 1, k < 0, n_sink < 0,
 * n_local < 0, n_sink + n_local > n, unknown key_type, short workspace. */
size_t topk_select_workspace_bytes(int rows, int n, int k, int key_type);
int topk_select(const void* keys, int key_type, int rows, int n, int k, int n_sink, int n_local,
                int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* topk_select_noalloc -- topk_select without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It calls no
 * allocating routine.  Its scratch is one static device array of
 * SDQ_TOPK_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends; the
 * first call on a device looks up that device's copy.  Every call on a GPU
 * shares that GPU's array, so calls that overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller.  Its contents on
 * entry do not matter (what must start at zero is cleared by a kernel).
 * Arguments, ordering, windows and output are those of topk_select.
 * Errors: those of topk_select; SDQ_EINVAL when
 * topk_select_workspace_bytes(rows, n, k, key_type) exceeds
 * SDQ_TOPK_NOALLOC_SCRATCH_BYTES (nothing is launched); SDQ_EHIP when the
 * scratch cannot be looked up on the current device. */
#define SDQ_TOPK_NOALLOC_SCRATCH_BYTES (16u << 20)
int topk_select_noalloc(const void* keys, int key_type, int rows, int n, int k, int n_sink,
                        int n_local, int32_t* idx_out, hipStream_t stream);

/* topk_select_block_max -- topk_select for float32 scores whose 64-key
 * block maxima are already known (fathom_scan writes them).  Same ordering,
 * windows and output as topk_select.  The k-th largest block maximum bounds
 * the k-th largest score from below, so only the blocks whose maximum
 * reaches it are read.  Needs no workspace.
 *   keys       float32 [rows][n], 16-byte aligned
 *   block_max  float32 [rows][n/64]: block_max[r][b] = max of keys[r][64b..64b+63]
 * Errors: as topk_select, plus SDQ_EINVAL if block_max is null, if n, n_sink
 * or n_local is not a multiple of 64, or n > 2^20. */
int topk_select_block_max(const float* keys, const float* block_max, int rows, int n, int k,
                          int n_sink, int n_local, int32_t* idx_out, hipStream_t stream);

/* topk_select_block_max_split -- topk_select_block_max with each row's
 * candidate gather spread over several workgroups (same sources, arguments,
 * ordering, windows and output).  The workgroups of a row derive the same
 * threshold, at most the k-th largest score, and each collects the keys that
 * reach it in its share of the row; their candidates meet in the workspace,
 * and a second launch selects exactly among them.  With group maxima the
 * threshold is the k-th largest maximum of the groups that lie wholly in the
 * competing range (each such group holds a competing block with that
 * maximum), and a workgroup reads only the block maxima of its own share;
 * without them, or with fewer than k such groups, every workgroup derives
 * the threshold from all of the row's block maxima.  Rows whose candidates
 * overflow take the exact row path, as in topk_select_block_max.
 *   block_max  as topk_select_block_max
 *   group_max  float32 [rows][ceil(n/64 / SDQ_GROUP_BLOCKS)], or NULL:
 *              group_max[r][j] = max of block_max[r][8j..8j+7] (of the
 *              blocks that exist), as fathom_scan writes it
 *   ws, ws_bytes  workspace of at least
 *             topk_select_block_max_split_workspace_bytes(rows, n) bytes,
 *             16-byte aligned; its contents on entry do not matter and calls
 *             on one workspace must not overlap.
 * Errors: those of topk_select_block_max, plus SDQ_EINVAL on a null or short
 * workspace or rows > 65535. */
size_t topk_select_block_max_split_workspace_bytes(int rows, int n);
int topk_select_block_max_split(const float* keys, const float* block_max, const float* group_max,
                                int rows, int n, int k, int n_sink, int n_local, int32_t* idx_out,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* hamming_scan -- dist[h][i] = popcount(sigs[h][i] XOR qsig[h]) in [0, 32]
 * (HashAttention study notes, sec. 2.2).
 *   sigs uint32 [H][n_cap] (rows of a growing cache, the first n scored);
 *   qsig uint32 [H];  dist uint8 [H][n] out
 * Errors: SDQ_EINVAL on null pointers, H < 1, n < 1, n > n_cap. */
int hamming_scan(const uint32_t* sigs, const uint32_t* qsig, int H, int n, int n_cap,
                 uint8_t* dist, hipStream_t stream);

/* hamming_scan_topk -- hamming_scan followed by topk_select(dist,
 * SDQ_KEY_U8_MIN, ...) in fewer launches (HashAttention study notes,
 * sec. 2.1: score every key, then keep the top-k).  On long rows the
 * distance kernel also writes the per-segment histograms the uint8 selection
 * reads, so the selection's first pass is not launched; otherwise the two
 * calls run one after the other.  dist and idx_out are identical to those of
 * the two separate calls (the selection is deterministic).
 *   sigs, qsig, H, n, n_cap, dist as hamming_scan (dist is written in full);
 *   k, n_sink, n_local, idx_out as topk_select with rows = H;
 *   ws, ws_bytes: at least topk_select_workspace_bytes(H, n, k,
 *                 SDQ_KEY_U8_MIN) bytes of device memory, owned by the caller
 * Errors: those of hamming_scan and topk_select. */
int hamming_scan_topk(const uint32_t* sigs, const uint32_t* qsig, int H, int n, int n_cap, int k,
                      int n_sink, int n_local, uint8_t* dist, int32_t* idx_out, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/* minmax_block_scan -- block scores against min/max summaries (OasisKV
 * review, Quest-style summaries):
 *   S[rg][b] = sum over the group's heads h and dims j of
 *              max(q[h][j] * bmin[rg][b][j], q[h][j] * bmax[rg][b][j])
 *   bmin, bmax fp16 [RG][nb_cap][d] (16-byte aligned; the first nb blocks
 *              of each row are scored);  q float32 [RG*H_grp][d];
 *   S float32 [RG][nb] out
 * Errors: SDQ_EINVAL on null pointers, RG < 1, H_grp < 1, nb < 1,
 * nb > nb_cap, d != 128, misaligned summaries. */
int minmax_block_scan(const uint16_t* bmin, const uint16_t* bmax, const float* q, int RG, int H_grp,
                      int nb, int nb_cap, int d, float* block_scores, hipStream_t stream);

/* gather_attend -- renormalised softmax attention over selected rows read by
 * index (HashAttention study notes, sec. 2.1 sparse output formula and
 * sec. 2.5 page-size-one reads):
 *   o[r][h] = sum_{i in I} e^{z_i} v_i / sum_{i in I} e^{z_i},
 *   z_i = softmax_scale * <q[r][h], K[r][kvh][i]>,  kvh = h / (H_q / H_kv)
 *   q     float32 [R][H_q][d]
 *   K, V  bf16 [R][H_kv][n_cap][d]: rows of n_cap tokens, the first n valid
 *   idx   int32 [R][H_sel][n_idx], H_sel = H_q if sets_per_query_head else
 *         H_kv (then the H_q/H_kv query heads of a group share the set).
 *         With block_tokens == 1 an entry is a row; with block_tokens > 1 it
 *         is a block id covering rows [b*block_tokens, (b+1)*block_tokens).
 *         Negative entries are padding and are skipped; entries must be
 *         distinct, and entries at or past n are skipped as well.
 *   out   float32 [R][H_q][d]; a set with no valid entry yields zeros.
 *   ws, ws_bytes  workspace of at least gather_attend_workspace_bytes() bytes
 *         (0 when every set fits one workgroup: then ws may be null).  It
 *         holds the partial results of sets split over several workgroups;
 *         its contents on entry do not matter.  Calls sharing a workspace
 *         must not overlap.
 * q, K and V must be 16-byte aligned; n < 2^23 (byte offsets within one
 * (request, KV head) slice fit 31 bits); H_q / H_kv in {1, 2, 4, 8} when sets
 * are shared; R * H_sel <= 65535.
 * Errors: SDQ_EINVAL on null pointers, R, H_q, H_kv, n, n_idx, block_tokens
 * < 1, n > n_cap, H_q % H_kv != 0, d != 128, the limits above, short
 * workspace. */
size_t gather_attend_workspace_bytes(int R, int H_q, int H_kv, int sets_per_query_head, int n_idx,
                                     int block_tokens, int d);
int gather_attend(const float* q, const uint16_t* K, const uint16_t* V, const int32_t* idx, int R,
                  int H_q, int H_kv, int sets_per_query_head, int n, int n_cap, int n_idx,
                  int block_tokens, int d, float softmax_scale, float* out, void* ws,
                  size_t ws_bytes, hipStream_t stream);

/* gather_attend_host_kv -- gather_attend with K and V left in host memory
 * (Fathom summary, offloaded setting: the KV rows live in host memory and
 * only the selected rows cross the host link, k * 512 bytes per set).  The
 * kernel reads the selected rows through the buffers' device mapping; no
 * staging copy is made.
 *   K_host, V_host  HOST pointers to pinned, device-mapped memory, bf16
 *                   [R][H_kv][n_cap][d] (16-byte aligned)
 *   everything else as gather_attend (q, idx, out and ws are device memory)
 * Errors: as gather_attend, and SDQ_EINVAL when K_host or V_host is not
 * pinned, device-mapped host memory. */
int gather_attend_host_kv(const float* q, const uint16_t* K_host, const uint16_t* V_host,
                          const int32_t* idx, int R, int H_q, int H_kv, int sets_per_query_head,
                          int n, int n_cap, int n_idx, int block_tokens, int d,
                          float softmax_scale, float* out, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Resident block pool (OasisKV review, core method and method steps)
 * --------------------------------------------------------------------- */

/* oasis_select -- KV selection of one step against a GPU-resident pool.
 * For every row r (a request's KV head): the predicted blocks P = pred[r]
 * are intersected with the pool resident[r] (S slots, block id or -1 for an
 * empty slot).  Hits keep their slot and get last_sel = step.  Predicted
 * blocks that are not resident (misses) are ordered by block_scores[r]
 * descending, equal scores to the lower block id; eviction targets (slots
 * whose block is not in P) are ordered empty slots first, then by last_sel
 * ascending, equal stamps to the lower slot.  The i-th miss is paired with the
 * i-th target for i < min(cap, misses, targets): the slot takes the block and
 * last_sel = step.
 *   pred          int32 [rows][K]  distinct block ids; entries outside
 *                 [0, nb) are ignored
 *   block_scores  float32 [rows][nb], not NaN
 *   resident, last_sel  int32 [rows][S]  in/out
 *   plan_slot, plan_block  int32 [rows][cap] out: the pairs in order, -1
 *                 padded (the transfer plan of oasis_fetch)
 *   n_fetch       int32 [rows] out: pairs made
 *   slots_out     int32 [rows][S] out, or NULL: s for every slot that holds a
 *                 block after the step, -1 otherwise (the index set of
 *                 gather_attend over the pool, in block units)
 * Limits: K <= 1024, S <= 1024, cap <= 1024, nb <= 65536.
 * Errors: SDQ_EINVAL on null pointers (pred and block_scores may be NULL when
 * K == 0, the plan when cap == 0), rows < 1 and the limits above. */
int oasis_select(const int32_t* pred, int K, const float* block_scores, int nb, int rows,
                 int32_t* resident, int32_t* last_sel, int S, int step, int cap,
                 int32_t* plan_slot, int32_t* plan_block, int32_t* n_fetch, int32_t* slots_out,
                 hipStream_t stream);

/* oasis_fetch -- carry out a transfer plan: block plan_block[r][i] of row r's
 * host cache is copied into slot plan_slot[r][i] of row r's pool, for both K
 * and V, read in place over the host link (OasisKV review: a UVA gather
 * kernel writes pinned host blocks straight into GPU-resident pages).  Pairs
 * with a slot or block out of range (the -1 padding) are skipped.
 *   K_host, V_host  HOST pointers to pinned, device-mapped memory, bf16
 *                   [rows][nb * block_tokens][d], 16-byte aligned
 *   K_pool, V_pool  bf16 [rows][S * block_tokens][d], 16-byte aligned
 * Errors: SDQ_EINVAL on null pointers, rows, nb, S or block_tokens < 1,
 * cap < 0, d != 128, more than 2^24 tokens per row, misalignment, host
 * memory the device cannot address. */
int oasis_fetch(const uint16_t* K_host, const uint16_t* V_host, const int32_t* plan_slot,
                const int32_t* plan_block, int rows, int cap, int nb, int block_tokens, int d,
                uint16_t* K_pool, uint16_t* V_pool, int S, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SDQ_H */
