/*
 * idx.h -- C ABI of the MI355X (gfx950) sparse-attention indexer library (libidx.so).
 *
 * The operation is the indexer of the GLM-5.3 indexer page
 * (sgl-amd-mono-upstream pull request 18).  For every decode or MTP-verify
 * row it scores each cached key of the row's request against the row's index
 * query and selects the row's exact top-k keys (Motivation; Modifications
 * item 0, the exact top-k check; items 2 and 3):
 *
 *   score[r][p] = sum_h w[r][h] * ReLU( s[p] * sum_d q[r][h][d] * k8[p][d] )
 *
 * with q the bf16 index query, w the bf16 head weights, k8 the key's OCP
 * FP8-E4M3FN code value and s its per-key f32 scale, for every logical
 * position p < n_keys[r].  The top-k set is the first k positions by score
 * descending, then position ascending (the page's definition of exactness);
 * the list is emitted in ascending position order, padded with -1 when a row
 * has fewer than k keys.
 *
 * Conventions shared by every entry point
 *  - Every array argument is a DEVICE pointer owned by the caller, except
 *    idx_problem.req_indptr, which is a HOST array.  The library allocates
 *    nothing on a call path and keeps no pointer after a call returns; buffers
 *    must stay alive until the stream has passed the call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is only enqueued; results follow stream order.
 *  - Return codes: IDX_OK, or one of the IDX_E* codes below.  Invalid
 *    arguments are rejected on the host before any HIP call.  No exception
 *    crosses the ABI and nothing is printed.
 *  - Device-resident values (n_keys, page ids) are checked by the kernels:
 *    an n_keys entry outside [0, max_keys] is clamped into range and a page
 *    id outside [0, num_pages) is replaced by page 0; either raises a sticky
 *    error bit in the workspace, read back with idx_device_status().
 *  - A workspace is used by one stream at a time; calls on distinct
 *    workspaces are independent.  It must be initialised once with
 *    idx_workspace_init(); a call leaves it usable by the next one.
 */
#ifndef IDX_H
#define IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Compiled shape (the GLM-5.3 indexer: 64 index heads of dimension 128,
 * pages of 64 keys; at most 4 rows of one request are scored together,
 * Modifications item 2). */
#define IDX_HEADS 64
#define IDX_DIM 128
#define IDX_PAGE_SIZE 64
#define IDX_KMAX 2048
#define IDX_GROUP_ROWS 4
#define IDX_MAX_REQ 256
#define IDX_MAX_KEYS (1 << 28)               /* keys a row at most (selection offsets stay 32-bit) */
#define IDX_NOALLOC_SCRATCH_BYTES (16u << 20) /* static scratch of idx_score_topk_noalloc, per device */
#define IDX_ABI_VERSION 3

/* Return codes. */
#define IDX_OK 0
#define IDX_EINVAL 1       /* null pointer, bad size/stride/alignment, k out of [1, IDX_KMAX], bad req_indptr */
#define IDX_EUNSUPPORTED 2 /* heads/dim/page size not the compiled ones, > IDX_MAX_REQ row groups,
                              max_keys > IDX_MAX_KEYS */
#define IDX_EWORKSPACE 3   /* workspace null or smaller than idx_workspace_bytes() */
#define IDX_EHIP 4         /* a HIP runtime call or launch failed; see idx_last_hip_error() */
#define IDX_EDEVICE 5      /* a sticky device-side error was found by idx_device_status() */
#define IDX_ESCRATCH 6     /* idx_score_topk_noalloc: the call needs more than IDX_NOALLOC_SCRATCH_BYTES */

/* Sticky device error bits (idx_device_status(), *detail). */
#define IDX_DERR_NKEYS 0x1u       /* an n_keys entry was outside [0, max_keys] */
#define IDX_DERR_PAGE 0x2u        /* a page id was outside [0, num_pages) */
#define IDX_DERR_WS 0x4u          /* the workspace was not initialised */
#define IDX_DERR_SELECT 0x10u     /* internal selection invariant failed (list count != k) */

typedef struct idx_problem {
  int32_t rows;              /* R >= 1 step rows */
  int32_t num_req;           /* 1 <= num_req; their row groups (below) at most IDX_MAX_REQ */
  const int32_t* req_indptr; /* HOST [num_req + 1]: request j owns rows [req_indptr[j], req_indptr[j+1]);
                                req_indptr[0] = 0, strictly increasing, req_indptr[num_req] = rows.
                                A request's rows are scored in groups of at most IDX_GROUP_ROWS
                                consecutive rows, each group reading the request's keys once;
                                at most IDX_MAX_REQ groups in all (sum of ceil(rows_j / 4)) */
  int32_t heads;             /* must be IDX_HEADS */
  int32_t dim;               /* must be IDX_DIM */
  int32_t page_size;         /* must be IDX_PAGE_SIZE */
  int32_t num_pages;         /* pages in the cache pool, >= 1 */
  int32_t max_pages;         /* columns of page_table, >= 1 */
  int32_t max_keys;          /* host bound on every n_keys[r]; 0 <= max_keys <= max_pages * page_size,
                                and max_keys <= IDX_MAX_KEYS (else IDX_EUNSUPPORTED) */
  const void* q;             /* bf16 [rows][heads][dim], finite, contiguous, 16-byte aligned */
  const void* w;             /* bf16 [rows][heads], finite, contiguous, 4-byte aligned */
  const uint8_t* k_cache;    /* E4M3FN codes [num_pages][page_size][dim], 16-byte aligned; no NaN
                                codes (0x7F, 0xFF) in the keys a row sees: a NaN score has no
                                place in the order and its row's list is unspecified */
  const float* k_scale;      /* f32 [num_pages][page_size], finite and >= 0, 16-byte aligned */
  const int32_t* page_table; /* int32 [rows][max_pages]: logical page j of row r is physical page
                                page_table[r][j]; rows of one request must hold the same entries for
                                the pages they use (the kernels walk the row with the most keys) */
  const int32_t* n_keys;     /* int32 [rows]: keys row r sees, 0 <= n_keys[r] <= max_keys */
  const int32_t* req_max_keys; /* HOST [num_req] or NULL: a bound on n_keys over each request's rows
                                  (<= max_keys).  Only sizes the launch: workgroups past a request's
                                  bound exit at once.  A row above its request's bound is clamped to
                                  it and raises IDX_DERR_NKEYS. */
} idx_problem;

/* ABI version (IDX_ABI_VERSION). */
int idx_abi_version(void);

/* Workspace size.  The selection's scratch is owned by the caller and allocated once,
 * outside the call path, as the indexer page sizes its select buffers once per runtime
 * (GLM-5.3 indexer page, Modifications item 3, "Scratch").  Sets *bytes to what every
 * entry point below needs for up to `rows` rows of up to `max_keys` keys and top-k size
 * k (one candidate block per row and chunk, plus a 256-byte header); the size grows
 * with rows and with max_keys, so one workspace serves every smaller call.
 * Returns IDX_OK; IDX_EINVAL (null bytes, rows outside [1, 2^24), max_keys < 0, k
 * outside [1, IDX_KMAX]); IDX_EUNSUPPORTED (max_keys > IDX_MAX_KEYS). */
int idx_workspace_bytes(int32_t rows, int32_t max_keys, int32_t k, size_t* bytes);

/* Zero the workspace and stamp it initialised (one device fill kernel on `stream`; no
 * host synchronisation).  Needed once per workspace: calls never leave state a later
 * call depends on, so it is not repeated between calls.  ws: device pointer, 256-byte
 * aligned; ws_bytes a multiple of 256 and >= 256.  Returns IDX_OK, IDX_EINVAL or
 * IDX_EHIP. */
int idx_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Scores only (steps S1-S4 of the path): the GLM-5.3 indexer page, Modifications item
 * 2 ("Scores": the bf16 query against every key of the request, scaled, ReLU'd and
 * head-summed in f32, each key read once for the up to 4 rows of a group; "Runs of
 * pages": the request's pages are streamed through LDS).  Writes scores[r * ld_scores + p]
 * (f32) for p < n_keys[r]; entries past n_keys[r] are left untouched.
 * ld_scores >= max(1, max_keys); scores 4-byte aligned, rows * ld_scores floats.
 * One launch on `stream`.  Returns IDX_OK, IDX_EINVAL, IDX_EUNSUPPORTED,
 * IDX_EWORKSPACE or IDX_EHIP; device-side errors are read with idx_device_status(). */
int idx_score(const idx_problem* p, float* scores, int64_t ld_scores,
              void* ws, size_t ws_bytes, void* stream);

/* Exact top-k over given scores (steps S5-S7): the GLM-5.3 indexer page, Modifications
 * item 3 (every row's exact top-2048) with item 0's definition of exactness (score
 * descending, then position).  For each row r, topk[r * k + i] (i < k) is the
 * ascending list of the first k positions p < n_keys[r] in that order, padded with -1
 * when n_keys[r] < k; scores compare as real numbers (-0 == +0) and must be finite.
 * scores: device f32 [rows][ld_scores]; n_keys: device int32 [rows] (values outside
 * [0, max_keys] are clamped and raise IDX_DERR_NKEYS); topk: device int32 [rows][k].
 * Any number of rows: launches of up to 1,024 rows each, in order on `stream`.
 * Returns IDX_OK, IDX_EINVAL, IDX_EUNSUPPORTED (max_keys > IDX_MAX_KEYS),
 * IDX_EWORKSPACE or IDX_EHIP. */
int idx_topk(const float* scores, int64_t ld_scores, const int32_t* n_keys,
             int32_t rows, int32_t max_keys, int32_t k, int32_t* topk,
             void* ws, size_t ws_bytes, void* stream);

/* The whole path (S1-S7): the GLM-5.3 indexer page, Modifications items 2 and 3 (a
 * request's rows scored together, then every row's exact top-k), exact in the sense
 * of item 0.  Two launches on `stream`: scoring, which also publishes each chunk's
 * candidates into the workspace, then one selection workgroup per row.  Writes the
 * scores exactly as idx_score() does and the lists exactly as idx_topk() over those
 * scores; 1 <= k <= IDX_KMAX; topk: device int32 [rows][k].  Returns as idx_score(). */
int idx_score_topk(const idx_problem* p, int32_t k, float* scores, int64_t ld_scores,
                   int32_t* topk, void* ws, size_t ws_bytes, void* stream);

/* Keys written in the same launch (the indexer page, Modifications item 2, on the keys a
 * launch writes: each verify row hands over its new index key as FP8 codes plus a scale,
 * and every scoring pass whose pages hold that position substitutes the key from that
 * hand-over for every row of the request, because the store to the cache may not have
 * reached memory when another pass reads the page).  Row r's key, codes[r][0..128)
 * (E4M3FN) and scales[r] (f32, finite, >= 0), takes logical position pos[r] of its
 * request: physical slot page_table[r][pos / 64] * 64 + pos % 64.  pos[r] = -1: the row
 * writes no key.  0 <= pos[r] < n_keys[r] otherwise (a row sees its own key); other
 * values raise IDX_DERR_NKEYS and the key is dropped by every row group of the request.
 * Device pointers; codes 16-byte aligned. */
typedef struct idx_new_keys {
  const uint8_t* codes;    /* E4M3FN [rows][128] */
  const float* scales;     /* f32 [rows] */
  const int32_t* pos;      /* int32 [rows] */
} idx_new_keys;

/* As idx_score_topk(), with every row's new key (idx_new_keys) in place: the scores are
 * those of the cache after the keys are written, and the launch also writes them into
 * p->k_cache and p->k_scale (which this call therefore modifies).  At most 16 rows a
 * request (else IDX_EUNSUPPORTED); nk null or misaligned: IDX_EINVAL. */
int idx_score_topk_append(const idx_problem* p, const idx_new_keys* nk, int32_t k, float* scores,
                          int64_t ld_scores, int32_t* topk, void* ws, size_t ws_bytes, void* stream);

/* As idx_score_topk(), and also each list as physical cache slots, the form the sparse
 * attention reads (the indexer page's selection stages its keys with their cache slots,
 * Modifications item 3, "Placing and resolving"): slots[r * k + i] =
 * page_table[r][p / 64] * 64 + p % 64 for the list entry p = topk[r * k + i] >= 0, and -1
 * where the list holds -1 (or where the page id lies outside the pool, which also raises
 * IDX_DERR_PAGE).  slots: device int32 [rows][k], distinct from topk.  Same launches;
 * the selection launch maps the list after writing it.  slots null or equal to topk:
 * IDX_EINVAL. */
int idx_score_topk_slots(const idx_problem* p, int32_t k, float* scores, int64_t ld_scores,
                         int32_t* topk, int32_t* slots, void* ws, size_t ws_bytes, void* stream);

/* As idx_score_topk_slots(), with the slots handed over as tagged words (the
 * GLM-5.3-Flash hand-offs page, Modifications item 3: the selection writes every
 * selected token together with the launch's tag, so a consumer polls the tokens
 * themselves, with no drain and no ready flag).  tagged[r * k + i] =
 * ((uint64_t)tag << 32) | (uint32_t)slot, slot as in idx_score_topk_slots() (-1 stored as
 * 0xFFFFFFFF), each word written by one 8-byte device-scope store after the row's list
 * is final.  A consumer on the same device that polls a word with device-scope loads
 * sees either an older word or the whole new one: a word is ready once its high half
 * equals `tag`.  The caller picks a tag no word holds yet (for example a launch
 * counter).  tagged: device uint64 [rows][k], 8-byte aligned.  topk is written as by
 * idx_score_topk().  Returns as idx_score_topk(). */
int idx_score_topk_tagged(const idx_problem* p, int32_t k, float* scores, int64_t ld_scores,
                          int32_t* topk, uint64_t* tagged, uint32_t tag, void* ws, size_t ws_bytes,
                          void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): idx_score_topk() with the candidate
 * blocks in a static scratch array of the library instead of a caller's workspace.
 * Each device holds its own IDX_NOALLOC_SCRATCH_BYTES-byte copy until the process
 * ends; the call allocates nothing and frees nothing.  The call's workspace need
 * (idx_workspace_bytes(rows, max_keys, k)) must fit it, else IDX_ESCRATCH.  Uses the
 * current device's scratch: `stream` must belong to the current device.  Calls on one
 * device share its scratch: calls whose executions overlap (other streams, other
 * threads) race and give undefined lists; calls in stream order are safe.  Nothing in
 * the scratch has to start at zero: every call writes every candidate word it reads.
 * Device-side errors (n_keys or page ids out of range) are clamped exactly as in
 * idx_score_topk() but not reported: there is no workspace for idx_device_status().
 * Returns IDX_OK, IDX_EINVAL, IDX_EUNSUPPORTED, IDX_ESCRATCH or IDX_EHIP. */
int idx_score_topk_noalloc(const idx_problem* p, int32_t k, float* scores, int64_t ld_scores,
                           int32_t* topk, void* stream);

/* Index-query preparation (the GLM-5.3 indexer page, Modifications item 2, on preparing
 * the query once a row: each row's index query gets its rotary embedding and the
 * Hadamard transform once and is stored in bf16; item 0's reference takes that query
 * computed in f32 with one rounding to bf16).  For every row r and head h, with
 * x = q_pre[r][h][:] (bf16 [rows][64][128]):
 *   1. RoPE on dimensions [0, rope_dim): pair i < rope_dim / 2 is (i, i + rope_dim / 2)
 *      (interleaved = 0) or (2 i, 2 i + 1) (interleaved = 1); its values (a, b) become
 *      (a c - b s, a s + b c) with c = cos_tab[r][i], s = sin_tab[r][i] (f32
 *      [rows][rope_dim / 2], the caller's rotation table for the row's position).
 *      Dimensions >= rope_dim pass through.
 *   2. The Hadamard transform: y = H x / sqrt(128), H the Sylvester Hadamard matrix,
 *      H[i][j] = (-1)^popcount(i & j).
 * q_out[r][h][:] = y rounded to bf16 (nearest, ties to even), computed in f32.  All
 * pointers are device pointers, 4-byte aligned; q_out must not overlap q_pre.
 * rope_dim is even in [0, 128] (cos_tab / sin_tab may be NULL when it is 0).  One
 * launch on `stream`.  Returns IDX_OK, IDX_EINVAL or IDX_EHIP. */
int idx_prep_query(const void* q_pre, const float* cos_tab, const float* sin_tab, int32_t rows,
                   int32_t rope_dim, int32_t interleaved, void* q_out, void* stream);

/* This library's device-side error channel (no page defines one): out-of-range n_keys
 * or page ids, an uninitialised workspace, a failed selection invariant.  Synchronises `stream`, reads and clears the workspace's sticky
 * error word.  Returns IDX_OK, IDX_EDEVICE (with *detail = IDX_DERR_* bits when detail
 * is not NULL), IDX_EINVAL (ws null or ws_bytes < 256) or IDX_EHIP. */
int idx_device_status(void* ws, size_t ws_bytes, void* stream, uint32_t* detail);

/* Static description of a return code. */
const char* idx_strerror(int code);

/* The last HIP error string seen by this thread (empty if none). */
const char* idx_last_hip_error(void);

/* SHA-256 (64 hex digits) of the sources and flags this library was built from, or
 * "unknown" for a build made without it. */
const char* idx_build_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H */
