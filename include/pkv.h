/*
 * pkv.h - C ABI of libpkv.so: paged-KV grouped-query decode attention with
 * split-KV parallelism for AMD Instinct MI355X (gfx950).
 *
 * The method (HALOps README, "Highlights"; HPC-Ops review, section "How the kernels
 * are organized around specific workload shapes"): decode attention over a paged
 * KV cache with grouped-query heads, BF16 or FP8 KV and a few speculative query
 * tokens; before every decode step each request's KV is cut into uniform tiles
 * that greedy bin-packing spreads over the workers; a split-KV kernel computes one
 * softmax-normalised partial result per tile, and a combine kernel merges them.
 *
 * One decode step through this ABI:
 *   1. pkv_plan_query + pkv_plan   (host; builds the work list from seq_lens)
 *   2. make items / worker_offsets / req_tile_base device-accessible (caller):
 *      copy them to device memory, or write them into mapped coherent pinned
 *      host memory that the kernels read directly
 *   3. pkv_decode_partial          (enqueued on a HIP stream)
 *   4. pkv_combine                 (enqueued on the same stream)
 * or, with no host work per step (e.g. inside a captured HIP graph):
 *   1. pkv_plan_device             (enqueued; same work list, built on the GPU from
 *                                   device seq_lens)
 *   2. pkv_decode_partial + pkv_combine as above, sized by the plan's capacity
 *
 * Conventions
 * - Every buffer, host or device, is allocated and owned by the caller. The
 *   library allocates nothing, keeps no state between calls and is thread-safe;
 *   the only per-thread state is the message behind pkv_last_error().
 * - Functions return a pkv_status (0 = success). Nothing aborts or throws across
 *   the ABI. Device entry points validate their host-visible arguments before any
 *   HIP call, then enqueue asynchronously and return without synchronising.
 * - The contents of device memory (lengths, block-table entries, work lists) are
 *   the caller's contract and are not read on the host. With the environment
 *   variable PKV_VALIDATE set (non-empty, not "0"), pkv_decode_partial,
 *   pkv_combine(_split), pkv_prefill, pkv_kv_append and pkv_block_sparse_compact
 *   first wait for their stream, copy those arrays to the host and check them, and
 *   return SEQ (a length below its minimum) or INVALID_ARG (a length past the block
 *   table, a block-table entry outside [0, num_pages), a work list that is not a
 *   plan of these lengths) with the detail in pkv_last_error, enqueuing nothing. A
 *   debugging aid: every such call is synchronous.
 * - Symbols used below: B = requests, Tq = query tokens per request (q_len),
 *   Hq / Hkv = query / kv heads, G = Hq / Hkv, M = G * Tq rows per work item,
 *   D = head_dim, P = page_size, T = tile tokens, W = workers.
 * - Layouts (row-major, last index fastest):
 *     q            bf16 [B, Tq, Hq, D]
 *     k/v_cache    bf16 or OCP e4m3fn bytes [num_pages, Hkv, P, D]
 *     k/v_scale    fp32 [num_pages, Hkv]: one scale per physical page and kv head
 *                  (FP8 with any P; with P = 64 a scale covers a 64-token tile)
 *     block_table  int32 [B, bt_stride]; entry (b, p) is the physical page of
 *                  request b's logical page p; only p < ceil(L_b / P) is read
 *     seq_lens     int32 [B]; L_b counts the Tq draft tokens, which sit at
 *                  positions L_b - Tq .. L_b - 1; draft row t sees keys 0 .. L_b-Tq+t
 *     out          bf16 [B, Tq, Hq, D]; lse_out fp32 [B, Tq, Hq] (natural log)
 *   Query head h reads kv head h / G. Tokens at or past L_b in a request's last
 *   page, block-table padding and unreferenced pages are never read.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 3

/* KV element formats. FP8 is OCP e4m3fn (bias 7, max 448, no infinities). */
enum pkv_kv_format { PKV_KV_BF16 = 0, PKV_KV_FP8_E4M3FN = 1 };

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad enum, ... */
  PKV_ERR_UNSUPPORTED = -2,  /* D not 64/128; P not a multiple of 16;
                                Hq % Hkv != 0; Tq not in [1, 4]; M > 64; tile not a
                                multiple of the quantum */
  PKV_ERR_ALIGNMENT = -3,    /* a device pointer is not 16-byte aligned */
  PKV_ERR_WORKSPACE = -4,    /* workspace smaller than pkv_workspace_bytes() */
  PKV_ERR_HIP = -5,          /* HIP runtime error; detail in pkv_last_error() */
  PKV_ERR_SEQ = -6           /* some L_b < 1 or L_b < Tq */
};

/* Version of this ABI (PKV_ABI_VERSION of the built library). */
int pkv_abi_version(void);

/* Static description of a status code; never NULL. */
const char* pkv_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none); the pointer is
 * valid until the next failing call on that thread. */
const char* pkv_last_error(void);

/*
 * Resolve the tile size and the plan's sizes for one decode step (host only).
 *
 * seq_lens_h : host int32 [batch]. tile_tokens: T, a multiple of the quantum
 * (P for bf16, lcm(P, 64) for fp8), or 0 for the automatic choice: among
 * quantum * 2^k <= 65536 the T minimising the bandwidth-sharing estimate
 *   kv * fluid(loads) + max_items_per_worker * 2^24 + N * M * (D + 1) * 8,
 * kv = 2 * D * eb bytes per token (eb = bytes per KV element), where with the
 * per-worker token loads sorted ascending l_1 <= ... <= l_W (l_0 = 0)
 *   fluid = sum_j (l_j - l_(j-1)) * max(W - j + 1, 160)
 * (while k workers are busy each streams at min(chip/k, chip/160)); ties go to the
 * larger T. num_workers: W >= 1
 * (see pkv_default_num_workers). Outputs: the resolved T, N = number of work
 * items, and the number of partial slots (= N).
 * Errors: INVALID_ARG (null pointer, batch < 0, W < 1), UNSUPPORTED (shape
 * rules above), SEQ (some L_b < max(1, q_len)).
 */
int pkv_plan_query(int batch, const int32_t* seq_lens_h, int q_len, int num_q_heads,
                   int num_kv_heads, int head_dim, int page_size, int kv_format,
                   int tile_tokens, int num_workers, int32_t* tile_tokens_out,
                   int64_t* num_items_out, int64_t* num_partials_out);

/*
 * Build the work list for tile size T and W workers (host only, deterministic).
 *
 * Work item (b, g, i) covers kv head g of request b, tokens [i*T, min(L_b, (i+1)*T)),
 * i < n_b = ceil(L_b / T); its cost is its token count. Items are placed longest
 * first (ties by (b, g, i) ascending), each on the least-loaded worker (ties to
 * the lowest index) - the greedy bin-packing of the HPC-Ops review.
 * Outputs (caller-allocated host arrays):
 *   items_h          int32 [N][4] = (b, g, i, slot), grouped by worker, each
 *                    worker's items in assignment order;
 *                    slot = Hkv * req_tile_base[b] + g * n_b + i
 *   worker_offsets_h int32 [W + 1]: worker w owns items [offsets[w], offsets[w+1])
 *   req_tile_base_h  int32 [batch + 1]: prefix sums of n_b
 * Errors: INVALID_ARG, SEQ (as pkv_plan_query).
 */
int pkv_plan(int batch, const int32_t* seq_lens_h, int q_len, int num_kv_heads,
             int tile_tokens, int num_workers, int32_t* items_h,
             int32_t* worker_offsets_h, int32_t* req_tile_base_h);

/* Recommended W for a device: compute units x resident decode workgroups per unit.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP (no such device). */
int pkv_default_num_workers(int device, int kv_format, int head_dim, int* out);

/* Workspace bytes for num_partials partial results of rows_per_partial (= M) rows
 * of D fp32 values plus one fp32 log-sum-exp per row; layout: o block at offset
 * 0, lse block at the next 256-byte boundary. Errors: INVALID_ARG. */
int pkv_workspace_bytes(int64_t num_partials, int rows_per_partial, int head_dim,
                        size_t* out);

/* Arguments of pkv_decode_partial. Pointers are device-accessible: device memory,
 * or (for the small plan arrays and seq_lens) mapped pinned host memory, which the
 * kernels then read directly without a host-to-device copy. */
typedef struct pkv_decode_args {
  size_t struct_size;             /* sizeof(pkv_decode_args) */
  const void* q;                  /* bf16 [B, Tq, Hq, D] */
  const void* k_cache;            /* [num_pages, Hkv, P, D], bf16 or e4m3fn */
  const void* v_cache;            /* same layout as k_cache */
  const float* k_scale;           /* fp32 [num_pages, Hkv]; NULL iff bf16 */
  const float* v_scale;           /* fp32 [num_pages, Hkv]; NULL iff bf16 */
  const int32_t* block_table;     /* int32 [B, bt_stride] */
  const int32_t* seq_lens;        /* int32 [B]; must equal the plan's seq_lens_h */
  const int32_t* items;           /* int32 [num_items][4] from pkv_plan (16-byte aligned) */
  const int32_t* worker_offsets;  /* int32 [num_workers + 1] from pkv_plan */
  const int32_t* req_tile_base;   /* int32 [B + 1] from pkv_plan */
  void* workspace;                /* pkv_workspace_bytes(num_partials, M, D) bytes */
  size_t workspace_bytes;
  int64_t num_items;
  int64_t num_partials;
  int64_t num_pages;
  int batch, q_len, num_q_heads, num_kv_heads, head_dim, page_size, bt_stride;
  int kv_format;                  /* enum pkv_kv_format */
  int tile_tokens;                /* resolved T of the plan */
  int num_workers;                /* W of the plan */
  float scale;                    /* softmax scale applied to q.k (e.g. 1/sqrt(D)) */
  /* ABI 2. Device int32 holding T; when non-NULL it replaces tile_tokens (which is
   * then not checked): pass info + 1 of pkv_plan_device. A struct_size that ends
   * before this field (an ABI 1 caller) means NULL. */
  const int32_t* tile_tokens_dev;
  /* ABI 2. Request split V >= 1 (0 and a struct_size ending before this field mean
   * 1): request b of the work list is part b % V of the caller's request b / V, and q
   * is [batch / V, Tq, V * num_q_heads, D]. Block-sparse decode uses V = Hkv with one
   * kv head per part (see pkv_block_sparse_compact); V = 1 is the layout above. */
  int request_split;
  /* ABI 3 (optional; a struct_size ending before these fields means NULL). When out is
   * non-NULL (bf16 [B, Tq, Hq, D], 16-byte aligned; request_split must be 1), the
   * items of requests cut into a single tile (L_b <= T) also write their rows' final
   * output and, if lse_out is non-NULL (fp32 [B, Tq, Hq]), log-sum-exp there, bit for
   * bit what pkv_combine would write for them. When every request of the plan is a
   * single tile (num_items == B * Hkv), the combine can then be skipped. */
  void* out;
  float* lse_out;
} pkv_decode_args;

/*
 * Split-KV partial attention (HALOps README, "Highlights": paged-KV decode attention
 * with GQA, BF16/FP8 KV, speculative decoding and split-KV; HPC-Ops review, "How the
 * kernels are organized around specific workload shapes": each uniform tile assigned
 * before the step yields a partial result that a separate kernel merges). One
 * persistent workgroup per worker walks its
 * items; for item (b, g, i) it gathers the tile's K/V pages through the block
 * table, runs an online softmax over the tile and writes, for each of the M rows
 * r = t*G + j (query token t, head g*G + j), the normalised partial output o
 * (fp32 [D]) and its log-sum-exp (fp32, natural log; -inf with o = 0 when the
 * causal mask hides every key of the tile from that row) into slot `slot`.
 * `stream` is a hipStream_t (NULL = null stream). Enqueue only; no sync.
 * Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT (q, caches, workspace must be
 * 16-byte aligned), WORKSPACE, HIP (launch failure).
 */
int pkv_decode_partial(const pkv_decode_args* args, void* stream);

/* Bytes of scratch pkv_plan_device needs for these arguments (the same values as
 * the pkv_plan_device call). With a fixed tile: 256 + 8 * batch * num_kv_heads.
 * With the automatic tile every candidate tile's plan is built at once, so it
 * holds, per candidate, its remainder-tile placements and a whole plan of up to
 * max_items items. Errors: INVALID_ARG. */
int pkv_plan_device_scratch_bytes(int batch, int num_kv_heads, int page_size, int kv_format,
                                  int tile_tokens, int num_workers, int64_t max_items,
                                  size_t* out);

/*
 * Device-side planner: the work list of pkv_plan_query + pkv_plan - the same
 * uniform tiles, longest-first greedy placement onto the workers and slot order,
 * bit for bit - built on the GPU from device seq_lens and enqueued on `stream`, so
 * a decode step needs no host work and can be captured in a HIP graph and replayed
 * with new lengths. The HPC-Ops review (section "How the kernels are organized
 * around specific workload shapes") has the tiles assigned before every decode
 * step; this entry point does that assignment on the device.
 *
 * tile_tokens: T (a multiple of the quantum) or 0 for the automatic rule of
 * pkv_plan_query, evaluated on the device and restricted to the candidate tiles
 * whose item count N fits max_items (the host's choice whenever that tile fits).
 * Arguments (device memory unless noted; caller-owned):
 *   seq_lens        int32 [batch]
 *   items           int32 [max_items][4], 16-byte aligned; rows (b, g, i, slot)
 *   worker_offsets  int32 [num_workers + 1]
 *   req_tile_base   int32 [batch + 1]
 *   info            int32 [4] = {status, T, N, most items on one worker}
 *   scratch         pkv_plan_device_scratch_bytes(...) bytes, 16-byte aligned;
 *                   contents need no initialisation
 * Limits: 1 <= num_workers <= 1024, batch <= 4096, 0 <= max_items <= INT32_MAX / 4,
 * tile_tokens <= 262144.
 * Returned errors (nothing enqueued): INVALID_ARG, UNSUPPORTED (shape rules, the
 * limits, tile not a multiple of the quantum), ALIGNMENT, WORKSPACE (scratch too
 * small), HIP. Errors found on the device go to info[0] with an empty plan (every
 * worker_offsets and req_tile_base entry 0: decode_partial then does nothing and
 * combine writes zeros with lse -inf): SEQ (some L_b < max(1, q_len)), UNSUPPORTED
 * (num_kv_heads * sum of L_b >= 2^36), WORKSPACE (N > max_items).
 * Then call pkv_decode_partial with num_items = num_partials = max_items,
 * tile_tokens_dev = info + 1 and a workspace for max_items partials, and
 * pkv_combine with num_partials = max_items.
 */
int pkv_plan_device(const int32_t* seq_lens, int batch, int q_len, int num_q_heads,
                    int num_kv_heads, int head_dim, int page_size, int kv_format,
                    int tile_tokens, int num_workers, int64_t max_items, int32_t* items,
                    int32_t* worker_offsets, int32_t* req_tile_base, int32_t* info,
                    void* scratch, size_t scratch_bytes, void* stream);

/*
 * Combine (HPC-Ops review, "How the kernels are organized around specific workload
 * shapes": a kernel of its own merges the split-KV partial results; HALOps README,
 * "Highlights": the reduction adapts to each request, so a request cut into one tile
 * is only normalised and cast). Log-sum-exp merge of the partials of each row (b, t, h):
 *   M* = max_i lse_i, w_i = exp(lse_i - M*), out = sum_i w_i o_i / sum_i w_i,
 *   lse_out = M* + ln sum_i w_i,   i = 0 .. n_b - 1 in order (deterministic),
 * n_b = req_tile_base[b+1] - req_tile_base[b] (device array). out is written in
 * bf16 (round to nearest even); lse_out may be NULL. Same workspace and stream as
 * pkv_decode_partial. Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT, WORKSPACE, HIP.
 */
int pkv_combine(const void* workspace, size_t workspace_bytes, int64_t num_partials,
                const int32_t* req_tile_base, int batch, int q_len, int num_q_heads,
                int num_kv_heads, int head_dim, void* out, float* lse_out, void* stream);

/* pkv_combine for a work list whose requests are split in V parts (request_split of
 * pkv_decode_args): out is [batch / V, Tq, V * num_q_heads, D] and lse_out
 * [batch / V, Tq, V * num_q_heads]. V = 1 is pkv_combine. Errors: as pkv_combine, and
 * INVALID_ARG when V < 1 or batch % V != 0. */
int pkv_combine_split(const void* workspace, size_t workspace_bytes, int64_t num_partials,
                      const int32_t* req_tile_base, int batch, int q_len, int num_q_heads,
                      int num_kv_heads, int head_dim, int request_split, void* out,
                      float* lse_out, void* stream);

/* Bytes of the device array pkv_decode_noalloc keeps on each GPU it runs on. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): one whole decode step,
 * pkv_decode_partial followed by pkv_combine on `stream`, with the split-KV partials
 * held in a library-owned device array of PKV_NOALLOC_SCRATCH_BYTES on each GPU
 * (kept until the process ends) instead of args->workspace, which is ignored (may be
 * NULL, with workspace_bytes 0). Every other argument is as for pkv_decode_partial
 * (args->struct_size must be sizeof(pkv_decode_args)); out and lse_out (may be NULL)
 * as for pkv_combine. The stream must belong to the current device. Makes no
 * allocation of any kind and runs no PKV_VALIDATE checks. All calls on one GPU share
 * that GPU's array: calls that overlap on one GPU (concurrent streams or threads)
 * race. Enqueue only; no sync.
 * Errors: as pkv_decode_partial and pkv_combine; WORKSPACE when
 * pkv_workspace_bytes(num_partials, M, D) exceeds PKV_NOALLOC_SCRATCH_BYTES (nothing
 * enqueued); HIP when the array's address cannot be obtained.
 */
int pkv_decode_noalloc(const pkv_decode_args* args, void* out, float* lse_out, void* stream);

/*
 * Block-sparse decode (the HALOps review's sparse attention: a precomputed block mask,
 * masked-out KV tiles skipped, per-tile FP8 scaling kept). The mask has one byte per
 * (request, kv head, logical page), nonzero = attended; the pages holding the step's
 * query tokens (positions L_b - Tq .. L_b - 1) are attended whatever their byte. Row t
 * of request b then attends to the keys j <= L_b - Tq + t whose page is attended.
 *
 * pkv_block_sparse_compact (enqueued) turns this into a dense one-kv-head problem of
 * batch * Hkv requests, request v = b * Hkv + g holding the attended pages of kv head
 * g of request b:
 *   block_table   device int32 [batch, bt_stride] (the caller's)
 *   seq_lens      device int32 [batch]
 *   block_mask    device uint8 [batch, Hkv, mask_stride], mask_stride >= bt_stride
 *   bt_out        device int32 [batch * Hkv, bt_stride]: row v lists phys * Hkv + g
 *                 of its attended pages in logical order (later entries untouched)
 *   seq_lens_out  device int32 [batch * Hkv]: attended tokens of row v (L_b minus
 *                 P per masked page); an invalid L_b is passed on unchanged
 * The one-kv-head problem reads the same cache viewed as [num_pages * Hkv, 1, P, D]
 * (scales as [num_pages * Hkv, 1]): plan it with num_kv_heads = 1, num_q_heads = G
 * and the seq_lens_out lengths (pkv_block_sparse_lengths computes them on the host),
 * run pkv_decode_partial with batch * Hkv requests, num_pages * Hkv pages, bt_out,
 * seq_lens_out and request_split = Hkv, then pkv_combine_split with request_split =
 * Hkv; out and lse_out keep the caller's [batch, Tq, Hq, ...] layout.
 * Errors: INVALID_ARG (null pointer, sizes), UNSUPPORTED (num_pages * Hkv >= 2^31
 * cannot be addressed), ALIGNMENT (int32 arrays), HIP.
 */
int pkv_block_sparse_compact(const int32_t* block_table, const int32_t* seq_lens,
                             const uint8_t* block_mask, int batch, int num_kv_heads,
                             int q_len, int page_size, int bt_stride, int mask_stride,
                             int64_t num_pages, int32_t* bt_out, int32_t* seq_lens_out,
                             void* stream);

/* Host twin of pkv_block_sparse_compact's lengths: lengths_out_h int32 [batch *
 * num_kv_heads] from host seq_lens and a host mask of the same layout, for planning on
 * the host. Errors: INVALID_ARG, SEQ (some L_b < max(1, q_len)). */
int pkv_block_sparse_lengths(int batch, const int32_t* seq_lens_h, const uint8_t* block_mask_h,
                             int num_kv_heads, int q_len, int page_size, int mask_stride,
                             int32_t* lengths_out_h);

/* Arguments of pkv_kv_append (all pointers device memory, caller-owned). */
typedef struct pkv_kv_append_args {
  size_t struct_size;             /* sizeof(pkv_kv_append_args) */
  const void* k_new;              /* bf16 [B, Tq, Hkv, D]: the step's new keys */
  const void* v_new;              /* bf16 [B, Tq, Hkv, D]: the step's new values */
  const void* q;                  /* bf16 [B, Tq, Hq, D] or NULL */
  void* q_out;                    /* bf16 [B, Tq, Hq, D]: rotated q (may equal q), or NULL */
  const float* rope_cos;          /* fp32 [max_pos, D/2] or NULL: no rotary embedding */
  const float* rope_sin;          /* fp32 [max_pos, D/2]; NULL iff rope_cos is */
  void* k_cache;                  /* [num_pages, Hkv, P, D], bf16 or e4m3fn, written */
  void* v_cache;
  float* k_scale;                 /* fp32 [num_pages, Hkv]; NULL iff bf16; read and written */
  float* v_scale;
  const int32_t* block_table;     /* int32 [B, bt_stride] */
  const int32_t* seq_lens;        /* int32 [B]; L_b counts the Tq new tokens */
  int64_t num_pages;
  int batch, q_len, num_q_heads, num_kv_heads, head_dim, page_size, bt_stride;
  int kv_format;                  /* enum pkv_kv_format */
  int max_pos;                    /* rows of the rotation tables; >= bt_stride * P */
} pkv_kv_append_args;

/*
 * Fused KV append: the step before decode attention (the HALOps README's fused
 * pre-processing of paged-KV decode; per-tile FP8 scaling as in the HALOps review),
 * in one kernel. Request b's Tq new tokens sit at positions L_b - Tq .. L_b - 1.
 * - Rotary embedding (when rope_cos is set), half-split form: for i < D/2, with
 *   c = rope_cos[pos, i], s = rope_sin[pos, i], x1 = x[i], x2 = x[i + D/2]:
 *   x[i] = x1*c - x2*s and x[i + D/2] = x2*c + x1*s, each product, sum and difference
 *   one IEEE float32 rounding; applied to the new k rows and, when q_out is set, to
 *   q (all heads) into q_out, rounded to bf16 (nearest even).
 * - bf16 cache: the (rotated) k rows and the v rows are stored at their positions
 *   (bit copies without rotation).
 * - fp8 cache: per page and kv head touched, K and V apart, with a = the largest
 *   |value| among the page's new rows: if the new rows start at the page's first
 *   slot the scale becomes a / 448 (1 if a == 0); else the page keeps its scale s
 *   while a / s <= 448, and otherwise takes a / 448 and re-encodes its earlier codes
 *   from their values code * s. Codes: nearest e4m3fn value (ties to the even code),
 *   saturating at +-448, sign kept. Divisions and products are IEEE float32.
 * Pages are written in place; a page must belong to one request. Enqueue only.
 * Errors: INVALID_ARG (null pointer, sizes, scales given iff fp8, one table only,
 * max_pos < bt_stride * P), UNSUPPORTED (shape rules), ALIGNMENT (16-byte rows and
 * caches, 4-byte tables), HIP.
 */
int pkv_kv_append(const pkv_kv_append_args* args, void* stream);

/*
 * Variable-length causal prefill over the paged cache (the HALOps README's
 * variable-length GQA prefill; the HPC-Ops launch article measures prefill for 128 to
 * 64K input tokens). A batch packs the query rows of B requests: q [total, Hq, D],
 * request b's rows at cu_q[b] .. cu_q[b+1]-1. Request b's n_b = cu_q[b+1] - cu_q[b]
 * query tokens are the last n_b of its kv_lens[b] cached tokens (a whole prompt, or a
 * chunk after a prefix), so its query t attends to keys j <= kv_lens[b] - n_b + t.
 * The cache, block table, GQA head mapping and FP8 scales are those of decode.
 *
 * Work items (host): one per (request, kv head, head group, 64-token query tile); a
 * head group is min(G, 4) query heads of the kv head (G must be 1, 2 or a multiple of
 * 4). pkv_prefill_plan lists them heaviest first (most keys, ties by (b, g, group,
 * tile)) as int32 [N][4] = (b, g, group, first token); pkv_prefill_plan_size gives N.
 * Errors: INVALID_ARG (null pointer, sizes, n_b > kv_len_b or n_b < 0), UNSUPPORTED
 * (G not 1, 2 or a multiple of 4).
 */
int pkv_prefill_plan_size(int batch, const int32_t* q_lens_h, int num_q_heads, int num_kv_heads,
                          int64_t* num_items_out);
int pkv_prefill_plan(int batch, const int32_t* q_lens_h, const int32_t* kv_lens_h, int num_q_heads,
                     int num_kv_heads, int32_t* items_h);

/* Arguments of pkv_prefill (pointers device-accessible, caller-owned). */
typedef struct pkv_prefill_args {
  size_t struct_size;             /* sizeof(pkv_prefill_args) */
  const void* q;                  /* bf16 [total, Hq, D] */
  const int32_t* cu_q;            /* int32 [B + 1] */
  const int32_t* kv_lens;         /* int32 [B] (each >= n_b) */
  const int32_t* block_table;     /* int32 [B, bt_stride] */
  const int32_t* items;           /* int32 [num_items][4] from pkv_prefill_plan, 16-byte aligned */
  const void* k_cache;            /* [num_pages, Hkv, P, D], bf16 or e4m3fn */
  const void* v_cache;
  const float* k_scale;           /* fp32 [num_pages, Hkv]; NULL iff bf16 */
  const float* v_scale;
  void* out;                      /* bf16 [total, Hq, D] */
  float* lse;                     /* fp32 [total, Hq] (natural log) or NULL */
  int64_t num_items;
  int64_t num_pages;
  int batch, num_q_heads, num_kv_heads, head_dim, page_size, bt_stride;
  int kv_format;                  /* enum pkv_kv_format */
  float scale;                    /* softmax scale */
} pkv_prefill_args;

/*
 * Enqueue the prefill kernel: one workgroup per work item; for its 64 query tokens and
 * head group it walks the causal key range in 32-key blocks with an online softmax
 * and writes each row's normalised output (bf16) and log-sum-exp. Every row of every
 * request must be covered by the items (pkv_prefill_plan's list). Device contents are
 * the caller's contract: an item outside the batch, or of a request with
 * kv_len < n_b or kv_len > bt_stride * P, is skipped and its rows are not written.
 * The softmax scale may be negative (taken exactly); a zero scale acts as the smallest
 * normal float. FP8 page scales must be positive. Enqueue only.
 * Errors: INVALID_ARG, UNSUPPORTED (D not 64/128, P not a multiple of 16,
 * G not 1, 2 or a multiple of 4), ALIGNMENT (q, out, caches, items 16 bytes),
 * HIP.
 */
int pkv_prefill(const pkv_prefill_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
