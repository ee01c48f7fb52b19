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
#define IDX_ABI_VERSION 2

/* Return codes. */
#define IDX_OK 0
#define IDX_EINVAL 1       /* null pointer, bad size/stride/alignment, k out of [1, IDX_KMAX], bad req_indptr */
#define IDX_EUNSUPPORTED 2 /* heads/dim/page size not the compiled ones, > IDX_MAX_REQ row groups */
#define IDX_EWORKSPACE 3   /* workspace null or smaller than idx_workspace_bytes() */
#define IDX_EHIP 4         /* a HIP runtime call or launch failed; see idx_last_hip_error() */
#define IDX_EDEVICE 5      /* a sticky device-side error was found by idx_device_status() */

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
  int32_t max_keys;          /* host bound on every n_keys[r]; 0 <= max_keys <= max_pages * page_size */
  const void* q;             /* bf16 [rows][heads][dim], contiguous, 16-byte aligned */
  const void* w;             /* bf16 [rows][heads], contiguous, 4-byte aligned */
  const uint8_t* k_cache;    /* E4M3FN codes [num_pages][page_size][dim], 16-byte aligned */
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

/* Bytes of workspace any entry point needs for up to `rows` rows of up to
 * `max_keys` keys and top-k size k.  Returns IDX_OK and sets *bytes, or
 * IDX_EINVAL. */
int idx_workspace_bytes(int32_t rows, int32_t max_keys, int32_t k, size_t* bytes);

/* Zero the workspace and stamp it initialised (a device fill kernel on
 * `stream`; no host synchronisation).  ws must be 256-byte aligned and
 * ws_bytes a multiple of 256 and >= 256. */
int idx_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Scores only: scores[r * ld_scores + p] for p < n_keys[r] (entries past
 * n_keys[r] are not written).  ld_scores >= max(1, max_keys). */
int idx_score(const idx_problem* p, float* scores, int64_t ld_scores,
              void* ws, size_t ws_bytes, void* stream);

/* Exact top-k over given scores: for each row r, topk[r * k + i] (i < k) is
 * the ascending list of the first k positions p < n_keys[r] by (score desc,
 * position asc), padded with -1; scores compare as real numbers (-0 == +0).
 * scores must be finite.  n_keys is a device array of `rows` entries. */
int idx_topk(const float* scores, int64_t ld_scores, const int32_t* n_keys,
             int32_t rows, int32_t max_keys, int32_t k, int32_t* topk,
             void* ws, size_t ws_bytes, void* stream);

/* Scoring and exact top-k in one call (two launches on `stream`: scoring with
 * candidate publication, then one selection workgroup per row): writes the
 * scores exactly as idx_score() does and the lists exactly as idx_topk() over
 * those scores. */
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
 * request (else IDX_EUNSUPPORTED). */
int idx_score_topk_append(const idx_problem* p, const idx_new_keys* nk, int32_t k, float* scores,
                          int64_t ld_scores, int32_t* topk, void* ws, size_t ws_bytes, void* stream);

/* As idx_score_topk(), and also each list as physical cache slots, the form the sparse
 * attention reads (the indexer page's selection stages cache slots, Modifications
 * item 3): slots[r * k + i] = page_table[r][p / 64] * 64 + p % 64 for
 * the list entry p = topk[r * k + i] >= 0, and -1 where the list holds -1 (or where the
 * page id lies outside the pool, which also raises IDX_DERR_PAGE).  slots: device
 * int32 [rows][k], distinct from topk.  Same launches; the selection launch maps the
 * list after writing it. */
int idx_score_topk_slots(const idx_problem* p, int32_t k, float* scores, int64_t ld_scores,
                         int32_t* topk, int32_t* slots, void* ws, size_t ws_bytes, void* stream);

/* Index-query preparation (the GLM-5.3 indexer page, Modifications item 2, "the query
 * once a row": each row's index query is roped and Hadamard-transformed once and
 * published in bf16; Modifications item 0: that transform runs in f32, then rounds to
 * bf16).  For every row r and head h, with x = q_pre[r][h][:] (bf16 [rows][64][128]):
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

/* Synchronise `stream`, read and clear the workspace's sticky device error.
 * Returns IDX_OK, IDX_EDEVICE (with *detail = IDX_DERR_* bits when detail is
 * not NULL), or IDX_EHIP. */
int idx_device_status(void* ws, size_t ws_bytes, void* stream, uint32_t* detail);

/* Static description of a return code. */
const char* idx_strerror(int code);

/* The last HIP error string seen by this thread (empty if none). */
const char* idx_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H */
