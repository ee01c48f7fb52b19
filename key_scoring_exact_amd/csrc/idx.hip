// libidx: MI355X (gfx950) sparse-attention indexer -- key scoring and exact top-k.
//
// The operation is the indexer of the GLM-5.3 indexer page (sgl-amd-mono-upstream
// pull request 18): every key of a request is scored against each row's bf16 index
// query (Modifications item 2: a request's rows scored together, each key read once),
// and each row's exact top-k is selected (item 3), exact in the sense of item 0:
// the first k positions by score descending, then position.
//
//   score[r][p] = sum_h w[r][h] * ReLU( s[p] * <q[r][h][:], k8[p][:]> )
//
// Two launches on the caller's stream cover the three entry points.
//
// Launch 1, scoring.  A workgroup (8 waves, two per SIMD) owns a chunk of P pages of
// one request group (at most 4 rows).  It loads the group's bf16 queries and head weights,
// then streams the chunk's key pages through registers into a ring of LDS page slots,
// widening each page's E4M3 codes to bf16 once at staging (exact: every finite E4M3 value
// is a bf16 value) and XOR-swizzling each key's 16-byte chunks so that the operand reads
// hit distinct banks.  Each wave holds the A operands of one row (64 heads) in registers
// and runs bf16 MFMA 32x32x16 over its tiles of 32 keys, in two accumulator chains.  FP8
// MFMA is not used: through an exact two-term E4M3 split of the query it costs the same
// matrix-core time, and its accumulation errs by about 2e-5 of the row's largest score
// against about 4e-8 for bf16.  The tile loop is software pipelined: the MFMAs of one tile
// are issued, then the epilogue of the previous tile (ReLU, head weights, f32 head sum,
// key scale) runs on the VALU while the matrix core works.  For each row longer than
// ALL_MAX keys, the workgroup also publishes every key of its chunk at or above a local
// threshold t_w (from a 128-bin histogram of the chunk's scores, so that at least m keys
// reach it), in position order, with a header word (t_w, count, overflow flag).
//
// Launch 2, selection: one workgroup per row.  A row of at most ALL_MAX keys loads
// all its scores into LDS.  A longer row gathers its chunks' candidates in position
// order and finds the exact k-th key T by radix select over the candidates at or
// above t* = max t_w: every such key is published, so when k of them are present no
// chunk can hide a key of the top k.  The selected positions are emitted in ascending
// order by one block scan, ties at T resolved by lowest position.  When that
// certificate fails, the chunks that may hide keys are re-read from the scores;
// anything beyond the LDS capacities takes an exact multi-pass radix select over the
// row's scores.  The kernel boundary orders the two launches: no workgroup waits on
// another.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "idx.h"

// Scratch of idx_score_topk_noalloc: the candidate blocks of one call, in place of a
// caller's workspace.  Each device that runs the library holds its own copy until the
// process ends.  Host code reaches it only through the address hipGetSymbolAddress
// returns for the current device (g_scratch below): in host code this name stands for a
// host-side shadow, not device memory.
static __device__ __align__(256) uint8_t scratch[IDX_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int H = IDX_HEADS;
constexpr int D = IDX_DIM;
constexpr int PS = IDX_PAGE_SIZE;
constexpr int GR = IDX_GROUP_ROWS;
constexpr int NT = 512;                 // threads per workgroup: 8 waves, two per SIMD
constexpr int NWAVE = NT / 64;
constexpr int PMAX = 8;                 // pages per workgroup at most
constexpr int CMAX = PMAX * PS;         // keys per chunk at most (512)
// pages in flight beyond the ones an iteration of the tile loop stages (TS / 2 pages an
// iteration, TS = waves a row): about four pages in registers in every case
__host__ __device__ constexpr int lookahead(int TS) { return TS == 2 ? 2 : 1; }
constexpr int ALL_MAX = 24576;          // rows up to this many keys select from all scores at once
constexpr int FIN_ENT = 12288;          // candidate capacity of a selecting workgroup
constexpr int CAP_MAX = 128;            // candidate slots per chunk and row
constexpr uint32_t WS_MAGIC = 0x1D5C0DE5u;

constexpr int MODE_SCORE = 1;           // compute scores (else read them from args.scores)
constexpr int MODE_PUBLISH = 2;         // publish each chunk's candidates for the selection launch
constexpr int MODE_NOMAGIC = 4;         // the workspace is the library's static scratch: no magic word to check

// LDS layout, scoring phase (bytes)
constexpr int NEW_MAX = 16;                                 // rows a request, when keys are written in the launch
constexpr int L_SC = 0;                                     // [GR][CMAX] f32 scores of the chunk
constexpr int L_KSC = L_SC + GR * CMAX * 4;                 // [PMAX][64] f32 key scales
constexpr int L_W = L_KSC + PMAX * PS * 4;                  // [GR][64] bf16 head weights
constexpr int L_PATCH = L_W + GR * H * 2;                   // [NEW_MAX][128 B] the request's new key codes
constexpr int L_KEYS = L_PATCH + NEW_MAX * D;               // ring of key pages widened to bf16, [slot][64 keys][256 B]
constexpr int PAGE16 = PS * D * 2;                          // one page in bf16
// The ring holds the pages of two iterations of the tile loop (TS / 2 pages an
// iteration, TS = waves a row), and the queries follow it: 8 / TS rows of 16 KiB.
__host__ __device__ constexpr int key_slots(int P, int TS) { return P < TS ? P : TS; }
__host__ __device__ constexpr int l_q(int P, int TS) { return L_KEYS + key_slots(P, TS) * PAGE16; }
__host__ __device__ constexpr int l_end(int P, int TS) { return l_q(P, TS) + (8 / TS) * H * D * 2; }
constexpr int L_SCORE_END = l_end(PMAX, 8) > l_end(PMAX, 2) ? l_end(PMAX, 8) : l_end(PMAX, 2);
// the publication's scratch, in the ring once the tile loop is done
constexpr int L_PHIST = L_KEYS;                             // [GR][128] u32 chunk histograms
constexpr int L_KST = L_PHIST + GR * 128 * 4;               // [GR][64] u32 keys of a bisection
static_assert(L_KST + GR * 64 * 4 <= L_KEYS + PAGE16, "publication scratch fits one ring slot");
static_assert(L_KEYS % 16 == 0 && l_end(PMAX, 4) <= L_SCORE_END, "layout");
// LDS layout, finishing phase
constexpr int HIST_WORDS = 4096 + 64;                       // one histogram: 4096 bins + 64 per-lane dummies
constexpr int L_HIST = 0;                                   // 2 histograms (low addresses: offsets fold into ds_add)
constexpr int L_MISC = L_HIST + 2 * HIST_WORDS * 4;         // 64 u32 scratch
constexpr int L_CAND = L_MISC + 64 * 4;                     // FIN_ENT u64 candidates + 64 dummies (or ALL_MAX u32 keys)
constexpr int BM_WORDS = 8 * NT;                            // chunk thresholds, then failing chunks or a list
constexpr int L_BM = L_CAND + (FIN_ENT + 64) * 8;           // [4 NT] chunk thresholds, [4 NT] failing chunks
constexpr int L_FIN_END = L_BM + BM_WORDS * 4;
static_assert(ALL_MAX % (4 * NT) == 0 && FIN_ENT % (4 * NT) == 0, "register segments of whole slot groups");
static_assert(ALL_MAX * 4 <= FIN_ENT * 8, "all-keys rows fit the candidate area");
static_assert(IDX_KMAX <= 4 * NT && IDX_KMAX + 64 <= BM_WORDS,
              "a list is four entries a thread; it and 64 dummy words fit the threshold area");
static_assert(L_CAND % 16 == 0, "16-byte candidate reads");
static_assert(CAP_MAX == 128, "a chunk's candidate block has at most four 32-slot groups");
static_assert(L_SCORE_END <= 160 * 1024 && L_FIN_END <= 160 * 1024, "LDS budget");

// workspace header (bytes)
constexpr int WS_MAGIC_OFF = 0;
constexpr int WS_ERR_OFF = 4;
constexpr int WS_HDR = 256;

// Stage timestamps (a build with -DIDX_STAMPS only): thread 0 of a workgroup writes the
// 100 MHz real-time counter at stage ends into 16 slots of its own record, in an area
// past the candidate blocks.  Scoring workgroup (x, y) owns record y * gridDim.x + x;
// selecting workgroup (x, y) owns record STAMP_SELECT + y * 4 + x.  Nothing else reads
// the area; the ordinary build compiles the stamps out.
constexpr int STAMP_SLOTS = 16;
constexpr int STAMP_SELECT = 8192;
constexpr int STAMP_RECORDS = STAMP_SELECT + 4 * IDX_MAX_REQ;
#ifdef IDX_STAMPS
constexpr uint64_t STAMP_BYTES = (uint64_t)STAMP_RECORDS * STAMP_SLOTS * 8;
#define STAMP(a, rec, id)                                                                              \
  do {                                                                                                 \
    if (threadIdx.x == 0)                                                                              \
      reinterpret_cast<uint64_t*>((a).ws + (a).off_stamps)[(uint64_t)(rec) * STAMP_SLOTS + (id)] =    \
          __builtin_amdgcn_s_memrealtime();                                                            \
  } while (0)
// the same through a record pointer (null: no stamp), for helpers without the arguments
#define STAMPP(p, id)                                                            \
  do {                                                                           \
    if (threadIdx.x == 0 && (p)) (p)[id] = __builtin_amdgcn_s_memrealtime();     \
  } while (0)
#else
constexpr uint64_t STAMP_BYTES = 0;
#define STAMP(a, rec, id) \
  do {                    \
  } while (0)
#define STAMPP(p, id) \
  do {                \
  } while (0)
#endif

struct KArgs {
  const uint8_t* q;         // bf16 [rows][64][128]
  const uint8_t* w;         // bf16 [rows][64]
  const uint8_t* kc;        // E4M3 [num_pages][64][128]
  const float* ks;          // f32 [num_pages][64]
  const int32_t* pt;        // int32 [rows][max_pages]
  const int32_t* nk;        // int32 [rows]
  float* scores;            // [rows][ld]: written (MODE_SCORE) or read
  int32_t* topk;            // [rows][k]
  uint8_t* ws;
  int64_t ld;
  int32_t rows, max_pages, max_keys, num_pages, k;
  int32_t chunk;            // keys per workgroup chunk (P * 64)
  int32_t chunk_shift;      // log2(chunk)
  int32_t mode;
  int32_t ent_stride;       // candidate blocks per row (>= chunks of a row that selects from candidates)
  uint64_t off_ent;
  uint32_t grp[IDX_MAX_REQ];// row0 | nrows << 24
  int32_t gmax[IDX_MAX_REQ];// host bound on the keys of each group's rows
  uint32_t req[IDX_MAX_REQ];// the group's request: its first row | its rows << 24 (with nw_pos)
  int32_t* slots;           // [rows][k] or null: the lists as physical cache slots
  // keys written in this launch (null nw_pos: none): row r's key (codes nw_codes[r],
  // scale nw_scales[r]) takes logical position nw_pos[r] (-1: none) of its request
  const uint8_t* nw_codes;  // E4M3 [rows][128]
  const float* nw_scales;   // f32 [rows]
  const int32_t* nw_pos;    // int32 [rows]
  uint8_t* kc_w;            // the cache, written
  float* ks_w;
  uint64_t* tagged;         // [rows][k] or null: the slots as tagged words, tag << 32 | slot
  uint32_t tag;
  uint64_t off_stamps;      // stage timestamps (IDX_STAMPS builds only)
};

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, off) (reinterpret_cast<T*>(smem + (off)))

// ---------------------------------------------------------------------------
// memory helpers
// ---------------------------------------------------------------------------
// A raw buffer resource over [base, base + bytes), bytes clamped to [0, 0x7FFFFFF0].  Every
// caller passes values the wave holds alike; they go through readfirstlane so that the
// resource sits in scalar registers also where the compiler cannot see that (arguments of
// a function that is not inlined), else each buffer instruction over it would become a
// loop over the lanes' distinct values.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0LL : (bytes < 0 ? 0 : bytes);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const int nn = __builtin_amdgcn_readfirstlane((int)n);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, nn, 0x00020000);
}

__device__ inline void raise_error(uint8_t* ws, uint32_t bits) {
  __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(ws + WS_ERR_OFF), bits, __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
}

// Monotone map of a finite f32 score to an unsigned key (larger score, larger key);
// -0 is first folded into +0 so that equal reals get equal keys.  Finite scores map
// to keys >= 0x00800000, so 0 never denotes a real score.
__device__ inline uint32_t radix_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);   // ~u if negative, else u | 2^31
}

__device__ inline int lane_id() { return (int)(threadIdx.x & 63); }
// the wave's index in the workgroup, as a wave-uniform (scalar) value
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Makes the given wave-uniform values live in scalar registers at this point: a kernel
// calls it on its arguments first, so that their loads go out together instead of one
// round trip behind each branch that first needs them.
template <typename T>
__device__ __forceinline__ void scalar_ready(const T& v) {
  asm volatile("" ::"s"(v));
}
template <typename... T>
__device__ __forceinline__ void scalars_ready(const T&... v) {
  (scalar_ready(v), ...);
}

// max(x, 0) of a float as one integer max of its bits: every negative float (and -0)
// is a negative int32, every positive float a positive one
__device__ inline float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// A lower bound t of the m-th largest of one value per lane (1 <= m <= 64), for values
// known to lie in [lo, hi] with at least m lanes >= lo: bisection over the bits below the
// common prefix of lo and hi, at most `bits` of them from the top, keeping #{v >= t} >= m.
// With every bit searched, t is the m-th largest itself.
__device__ __forceinline__ uint32_t wave_kth_bound(uint32_t v, int m, uint32_t lo, uint32_t hi, int bits) {
  const uint32_t diff = lo ^ hi;
  if (diff == 0u) return lo;
  const int top = 31 - __clz(diff);
  uint32_t t = top == 31 ? 0u : lo & ~((2u << top) - 1u);
  const int last = top - bits + 1 > 0 ? top - bits + 1 : 0;
  for (int b = top; b >= last; --b) {
    const uint32_t c = t | (1u << b);
    if ((int)__popcll(__ballot(v >= c)) >= m) t = c;
  }
  return t;
}

// ---------------------------------------------------------------------------
// wave and workgroup primitives on DPP (VALU lane moves; no LDS round trips)
// ---------------------------------------------------------------------------
// DPP controls: row_shr:n = 0x110 + n (within rows of 16 lanes), row_bcast:15 = 0x142
// (lane 15 of each row to the next row), row_bcast:31 = 0x143 (lane 31 to rows 2, 3).
// A lane whose source is outside its row, or whose row is masked off, keeps `old`.
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROWMASK, 0xF, false);
}

__device__ __forceinline__ int wave_incl_scan(int x) {
  uint32_t v = (uint32_t)x;
  v += dpp<0x111>(0u, v);
  v += dpp<0x112>(0u, v);
  v += dpp<0x114>(0u, v);
  v += dpp<0x118>(0u, v);
  v += dpp<0x142, 0xA>(0u, v);
  v += dpp<0x143, 0xC>(0u, v);
  return (int)v;
}

// within each row of 16 lanes, lane 15 ends up holding the row's max / min / sum (lanes
// shifted in from outside the row read the operation's identity, so each step is one
// DPP-modified max, min or add)
__device__ __forceinline__ uint32_t row_max(uint32_t v) {
  v = max(v, dpp<0x111>(0u, v));
  v = max(v, dpp<0x112>(0u, v));
  v = max(v, dpp<0x114>(0u, v));
  v = max(v, dpp<0x118>(0u, v));
  return v;
}
__device__ __forceinline__ uint32_t row_min(uint32_t v) {
  v = min(v, dpp<0x111>(0xFFFFFFFFu, v));
  v = min(v, dpp<0x112>(0xFFFFFFFFu, v));
  v = min(v, dpp<0x114>(0xFFFFFFFFu, v));
  v = min(v, dpp<0x118>(0xFFFFFFFFu, v));
  return v;
}
__device__ __forceinline__ uint32_t row_sum(uint32_t v) {
  v += dpp<0x111>(0u, v);
  v += dpp<0x112>(0u, v);
  v += dpp<0x114>(0u, v);
  v += dpp<0x118>(0u, v);
  return v;
}
__device__ __forceinline__ uint32_t rl(uint32_t v, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)v, l); }
// wave-uniform results
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row_max(v);
  return max(max(rl(v, 15), rl(v, 31)), max(rl(v, 47), rl(v, 63)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = row_min(v);
  return min(min(rl(v, 15), rl(v, 31)), min(rl(v, 47), rl(v, 63)));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v = row_sum(v);
  return rl(v, 15) + rl(v, 31) + rl(v, 47) + rl(v, 63);
}

// Exclusive scan over the workgroup; `tmp` is NWAVE ints of LDS (16-byte aligned).
// Every thread must call.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int l = lane_id(), wv = wave_id();
  const int x = wave_incl_scan(v);
  if (l == 63) tmp[wv] = x;
  __syncthreads();
  const v4i a = reinterpret_cast<const v4i*>(tmp)[0];
  const v4i b = reinterpret_cast<const v4i*>(tmp)[1];
  const int t[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; i++) {
    before += (i < wv) ? t[i] : 0;
    tot += t[i];
  }
  __syncthreads();
  if (total) *total = tot;
  return x - v + before;
}

// Histogram increment of one key per lane (when `m`), aggregated over the wave: up to
// four rounds each add the count of the bin of the first lane still pending with one
// atomic, then the rest add one each.  Radix digits of nearby or tied scores pile into
// a few bins, and serialised LDS atomics on one address are the cost to avoid.
__device__ inline void hist_add(uint32_t* hist, bool m, uint32_t bin) {
  uint64_t act = __ballot(m);
#pragma unroll
  for (int round = 0; round < 4; round++) {
    if (act == 0) return;
    const int first = __ffsll((unsigned long long)act) - 1;
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
    const uint64_t sb = __ballot(bin == lb) & act;
    if (lane_id() == first) atomicAdd(&hist[lb], (uint32_t)__popcll(sb));
    act &= ~sb;
  }
  if ((act >> lane_id()) & 1ull) atomicAdd(&hist[bin], 1u);
}

// Radix digit search: the digit d of hist[0 .. nbins) (nbins a power of two, <= 4096)
// holding the rem-th largest remaining key, counting from the top bin.  Thread t scans
// bins [nbins - 8 t - 8, nbins - 8 t).  Writes misc[8] = d, misc[9] = rem left within
// d, misc[10] = count of d.  Every thread must call; two barriers.
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nbins, int rem, int* misc) {
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int base = nbins - 8 * (tid + 1);
  uint32_t h[8];
  if (base >= 0) {
    const v4i a = *reinterpret_cast<const v4i*>(hist + base);
    const v4i b = *reinterpret_cast<const v4i*>(hist + base + 4);
    h[0] = a[0]; h[1] = a[1]; h[2] = a[2]; h[3] = a[3];
    h[4] = b[0]; h[5] = b[1]; h[6] = b[2]; h[7] = b[3];
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) h[i] = (base + i >= 0) ? hist[base + i] : 0u;
  }
  int c = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) c += (int)h[i];
  const int incl = wave_incl_scan(c);
  if (lane == 63) misc[wv] = incl;
  __syncthreads();
  const v4i ta = reinterpret_cast<const v4i*>(misc)[0];
  const v4i tb = reinterpret_cast<const v4i*>(misc)[1];
  const int t[8] = {ta[0], ta[1], ta[2], ta[3], tb[0], tb[1], tb[2], tb[3]};
  int before = incl - c;
#pragma unroll
  for (int i = 0; i < NWAVE; i++) before += (i < wv) ? t[i] : 0;
  if (c > 0 && before < rem && rem <= before + c) {
    int r = rem - before, d = base + 7, dc = (int)h[7];
#pragma unroll
    for (int i = 7; i >= 0; i--) {
      if (r <= (int)h[i]) { d = base + i; dc = (int)h[i]; break; }
      r -= (int)h[i];
    }
    misc[8] = d;
    misc[9] = r;
    misc[10] = dc;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Exact top-k threshold of the keys held in registers across the workgroup: thread t
// holds kr[0 .. S) (S a multiple of 4); a zero key is absent, cnt keys are present and
// all of them lie in [lo, hi].  Both histogram buffers (hist: 2 x HIST_WORDS words) must
// be clear on entry and are left dirty.  Returns false if cnt < k.  Otherwise the top k
// (score descending, then position) are exactly: every key >= *Tge, and, when *rem > 0,
// also the first *rem keys equal to Tge - 1 in position order.
//
// First pass: a histogram of 4096 bins linear in the score over [lo, hi], bin(key) =
// floor(score * s - lo_score * s) with s = 4096 / (hi_score - lo_score), the product and
// difference rounded once (an fma), clamped to [0, 4095].  A once-rounded function of a
// real that is monotone in the score is monotone, so every key of a higher bin is larger
// than every key of a lower one, and the bin d holding the k-th largest key leaves r =
// (k minus the keys above d) to choose inside it.  Scores of one row cluster far below
// the f32 exponent scale, so a bin this fine holds a few keys: they are listed and wave
// 0 finds the r-th largest exactly.  A bin of more than 64 keys (ties, or a degenerate
// spread) falls back to radix passes over the keys in [min, max] of that bin, in digits
// of up to 12 bits below the common prefix.  Absent keys and keys outside the range in
// play go to per-lane dummy words past the bins (with SPARSE, for slots mostly absent,
// they are skipped instead).  Every thread must call.
// ---------------------------------------------------------------------------
// the f32 score a key encodes (the inverse of radix_key for keys of finite scores)
__device__ __forceinline__ float key_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// min and max over the workgroup.  Every thread must call.
__device__ __forceinline__ void block_min_max(uint32_t& mn, uint32_t& mx, int* misc) {
  const int lane = lane_id(), wv = wave_id();
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  uint32_t* red = reinterpret_cast<uint32_t*>(misc) + 16;
  if (lane == 0) {
    red[wv] = mn;
    red[NWAVE + wv] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NWAVE; i++) {
    mn = min(mn, red[i]);
    mx = max(mx, red[NWAVE + i]);
  }
  __syncthreads();
}

// Sum over the workgroup (wave-uniform result).  Every thread must call.
__device__ __forceinline__ uint32_t block_sum(uint32_t v, int* misc) {
  v = wave_sum_u32(v);
  if (lane_id() == 0) misc[wave_id()] = (int)v;
  __syncthreads();
  const v4i a = reinterpret_cast<const v4i*>(misc)[0];
  const v4i b = reinterpret_cast<const v4i*>(misc)[1];
  __syncthreads();
  return (uint32_t)(a[0] + a[1] + a[2] + a[3] + b[0] + b[1] + b[2] + b[3]);
}

// zero the 4096 bins of both histogram buffers (no barrier)
__device__ __forceinline__ void clear_hist(uint32_t* hist) {
  const v4i z = {0, 0, 0, 0};
  const int t = threadIdx.x;
#pragma unroll
  for (int b = 0; b < 2; b++) {
    v4i* h4 = reinterpret_cast<v4i*>(hist + b * HIST_WORDS);
    h4[t] = z;
    h4[t + NT] = z;
  }
}

template <int SMAX, bool SPARSE = false>
__device__ __forceinline__ bool kth_select(const uint32_t (&kr)[SMAX], int S, int cnt, uint32_t lo, uint32_t hi,
                                           int k, uint32_t* hist, int* misc, uint32_t* Tge_out, int* rem_out,
                                           uint64_t* stp = nullptr) {
  static_assert(SMAX % 4 == 0, "slot groups of 4");
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  if (cnt < 0 && lo == hi) {                          // an unknown count is needed here: count the keys
    uint32_t c0 = 0;
#pragma unroll
    for (int j = 0; j < SMAX; j++) c0 += (j < S && kr[j] != 0u) ? 1u : 0u;
    cnt = (int)block_sum(c0, misc);
  }
  if (cnt >= 0 && cnt < k) return false;
  if (lo == hi) {  // every key equal: the first k of them (all of them when cnt == k)
    *Tge_out = cnt == k ? lo : lo + 1u;
    *rem_out = cnt == k ? 0 : k;
    return true;
  }
  const uint32_t dummy = 4096u + (uint32_t)lane;
  uint32_t klo = lo, khi = hi;                        // keys in play: [klo, khi]
  int rem = k, buf = 0;

  // ---- linear pass: 4096 bins linear in the score over [lo, hi], bin(key) =
  // floor(score * s - lo_score * s) with s = 4096 / (hi_score - lo_score), the product and
  // difference rounded once (an fma), clamped to [0, 4095]: a once-rounded monotone function
  // of the score, so every key of a higher bin is larger than every key of a lower one
  const float fmin = key_float(lo);
  const float span = key_float(hi) - fmin;
  const float scale = 4096.0f / span;
  if (span <= 3.0e38f && scale <= 3.0e38f) {          // both finite (false for inf, NaN)
    const float off = -fmin * scale;
    uint32_t idx[SMAX];
    if (tid == 0) {
      misc[10] = -1;                                  // no bin found (fewer than k keys)
      misc[11] = 0;                                   // list counter
    }
#pragma unroll
    for (int g = 0; g < SMAX / 4; g++) {
      if (g * 4 < S) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int j = g * 4 + jj;
          const uint32_t key = kr[j];
          const uint32_t b = min(__float2uint_rz(fmaf(key_float(max(key, lo)), scale, off)), 4095u);
          idx[j] = key != 0u ? b : dummy;
          // most slots absent (SPARSE): count only the present keys; else every slot,
          // the absent ones into the lane's dummy word, without a branch
          if (!SPARSE) atomicAdd(&hist[idx[j]], 1u);
          else if (key != 0u) atomicAdd(&hist[b], 1u);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; jj++) idx[g * 4 + jj] = dummy;
      }
    }
    __syncthreads();
    STAMPP(stp, 6);
    find_digit(hist, 4096, rem, misc);
    STAMPP(stp, 7);
    const uint32_t d = (uint32_t)misc[8];
    const int r = misc[9];
    const int c = misc[10];
    if (c < 0) return false;                          // fewer than k keys
    if (c == 1) {
      // bin d holds one key, the k-th: every key above it and it are in (r == 1)
#pragma unroll
      for (int g = 0; g < SMAX / 4; g++) {
        if (g * 4 >= S) break;
#pragma unroll
        for (int jj = 0; jj < 4; jj++)
          if (idx[g * 4 + jj] == d) misc[12] = (int)kr[g * 4 + jj];
      }
      __syncthreads();
      *Tge_out = (uint32_t)misc[12];
      *rem_out = 0;
      return true;
    }
    if (c <= 64) {
      // the c keys of bin d into a list (the dummy words of the second buffer), then the
      // r-th largest of them on wave 0
      uint32_t* lst = hist + HIST_WORDS + 4096;
#pragma unroll
      for (int g = 0; g < SMAX / 4; g++) {
        if (g * 4 >= S) break;
#pragma unroll
        for (int jj = 0; jj < 4; jj++)
          if (idx[g * 4 + jj] == d) lst[atomicAdd(&misc[11], 1)] = kr[g * 4 + jj];
      }
      STAMPP(stp, 8);
      __syncthreads();
      if (wv == 0) {
        // the r-th largest listed key: the x with #{> x} < r <= #{>= x} (lanes past c
        // hold 0, below every key)
        const uint32_t v = lane < c ? lst[lane] : 0u;
        uint32_t T = 0u;
        int gt = 0, eq = 0;
        for (int i2 = 0; i2 < c; i2++) {
          const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)v, i2);
          const int g2 = (int)__popcll(__ballot(v > x));
          const int e2 = (int)__popcll(__ballot(v == x));
          if (g2 < r && r <= g2 + e2) {
            T = x;
            gt = g2;
            eq = e2;
            break;
          }
        }
        if (lane == 0) {
          // keys above T are all selected; r - gt of the eq keys equal to T
          misc[12] = (int)(r - gt == eq ? T : T + 1u);
          misc[13] = r - gt == eq ? 0 : r - gt;
        }
      }
      STAMPP(stp, 10);
      __syncthreads();
      *Tge_out = (uint32_t)misc[12];
      *rem_out = misc[13];
      return true;
    }
    // a crowded bin: its key range, then radix passes over it
    uint32_t bmn = 0xFFFFFFFFu, bmx = 0u;
#pragma unroll
    for (int g = 0; g < SMAX / 4; g++) {
      if (g * 4 >= S) break;
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const bool in = idx[g * 4 + jj] == d;
        const uint32_t key = kr[g * 4 + jj];
        bmn = min(bmn, in ? key : 0xFFFFFFFFu);
        bmx = max(bmx, in ? key : 0u);
      }
    }
    block_min_max(bmn, bmx, misc);
    klo = bmn;
    khi = bmx;
    rem = r;
    if (r == c) {                                     // all of bin d
      *Tge_out = klo;
      *rem_out = 0;
      return true;
    }
    if (klo == khi) {                                 // r of the c equal keys of bin d
      *Tge_out = klo + 1u;
      *rem_out = r;
      return true;
    }
    buf = 1;                                          // still clear
  }

  // ---- radix passes over the keys in [klo, khi]
  const int top = 31 - __clz(klo ^ khi);             // highest bit that differs
  uint32_t mask = (top == 31) ? 0u : ~((2u << top) - 1u);
  uint32_t prefix = klo & mask;
  const uint32_t span_k = khi - klo;
  const int nb = top + 1;                             // bits left to resolve
  const int npass = (nb + 11) / 12;
  const int wdef = (nb + npass - 1) / npass;
  int shift = nb;
  while (true) {
    const int width = wdef < shift ? wdef : shift;
    shift -= width;
    uint32_t* h = hist + buf * HIST_WORDS;
#pragma unroll
    for (int g = 0; g < SMAX / 4; g++) {
      if (g * 4 >= S) break;
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const uint32_t key = kr[g * 4 + jj];
        const uint32_t dg = __builtin_amdgcn_ubfe(key, (uint32_t)shift, (uint32_t)width);
        const bool in = key - klo <= span_k && (key & mask) == prefix;   // absent keys wrap out
        if (!SPARSE) atomicAdd(&h[in ? dg : dummy], 1u);
        else if (in) atomicAdd(&h[dg], 1u);
      }
    }
    {
      // the other buffer is free: clear it for the next pass
      const v4i z = {0, 0, 0, 0};
      v4i* h4 = reinterpret_cast<v4i*>(hist + (buf ^ 1) * HIST_WORDS);
      h4[tid] = z;
      h4[tid + NT] = z;
    }
    __syncthreads();
    find_digit(h, 1 << width, rem, misc);
    const uint32_t d = (uint32_t)misc[8];
    const int r = misc[9];
    const int c = misc[10];
    const uint32_t dmask = (1u << width) - 1u;
    prefix |= d << shift;
    mask |= dmask << shift;
    if (c == r) {
      // every key of this digit is selected: the top k are exactly the keys >= prefix
      // (and >= klo: keys below klo belong to lower bins)
      *Tge_out = max(prefix, klo);
      *rem_out = 0;
      return true;
    }
    if (shift == 0) {
      // r of the c keys equal to prefix, in position order
      *Tge_out = prefix + 1u;
      *rem_out = r;
      return true;
    }
    rem = r;
    buf ^= 1;
  }
}

// Emission of the top k in segment order (thread t's slots j < S precede thread t + 1's;
// the caller lays positions out ascending in that order; absent slots hold key 0): a
// key is selected when key >= Tge, or, when rem > 0, key == Tge - 1 and it is among
// the first rem such keys.  Each thread stores its selected positions pr[j] straight
// to their ranks in out[0 .. k) (a contiguous run a thread, the runs in thread order).
// Unselected slots store past the buffer resource, which drops them; with MASKED they
// store nothing (the lane is masked off), which is faster where every slot of a thread
// holds a key (rows selected from all their scores).  Returns the number selected.
// Every thread must call.
template <int SMAX, bool MASKED = false>
__device__ __forceinline__ int emit_segments(const uint32_t (&kr)[SMAX], const uint32_t (&pr)[SMAX], int S,
                                             uint32_t Tge, int rem, int32_t* out, int k, int* misc) {
  const uint32_t T = Tge - 1u;
  int gt = 0, eq = 0;
#pragma unroll
  for (int g = 0; g < SMAX / 4; g++) {
    if (g * 4 >= S) break;
#pragma unroll
    for (int jj = 0; jj < 4; jj++) gt += kr[g * 4 + jj] >= Tge ? 1 : 0;
  }
  if (rem > 0) {
#pragma unroll
    for (int g = 0; g < SMAX / 4; g++) {
      if (g * 4 >= S) break;
#pragma unroll
      for (int jj = 0; jj < 4; jj++) eq += kr[g * 4 + jj] == T ? 1 : 0;
    }
  }
  int tot;
  const int packed = block_excl_scan(gt | (eq << 16), misc, &tot);
  const int before_gt = packed & 0xFFFF, before_eq = packed >> 16;
  // stores without branches: an unselected slot stores past the buffer resource, which
  // drops it
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(out, (int64_t)k * 4);
  if (rem == 0) {
    int o = before_gt;
#pragma unroll
    for (int g = 0; g < SMAX / 4; g++) {
      if (g * 4 >= S) break;
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const bool sel = kr[g * 4 + jj] >= Tge;
        if (MASKED) {
          if (sel) __builtin_amdgcn_raw_buffer_store_b32(pr[g * 4 + jj], rout, o * 4, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(pr[g * 4 + jj], rout, sel ? o * 4 : 0x7FFFFFF0, 0, 0);
        }
        o += sel ? 1 : 0;
      }
    }
  } else {
    int o = before_gt + (before_eq < rem ? before_eq : rem);
    int er = before_eq;
#pragma unroll
    for (int g = 0; g < SMAX / 4; g++) {
      if (g * 4 >= S) break;
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const uint32_t key = kr[g * 4 + jj];
        const bool e = key == T;
        const bool sel = key >= Tge || (e && er < rem);
        er += e ? 1 : 0;
        if (MASKED) {
          if (sel) __builtin_amdgcn_raw_buffer_store_b32(pr[g * 4 + jj], rout, o * 4, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(pr[g * 4 + jj], rout, sel ? o * 4 : 0x7FFFFFF0, 0, 0);
        }
        o += sel ? 1 : 0;
      }
    }
  }
  const int tg = tot & 0xFFFF, te = tot >> 16;
  const int got = tg + (te < rem ? te : rem);
  return got;
}

// Emission of the top k from slots held piece-major: thread t holds pieces u NT + t
// (u < np, np uniform) of W slots each, kr/pr[W u + h], and the slots run in the order
// (u, t, h), which the caller makes ascending in position.  Selection as in
// emit_segments: key >= Tge, or key == Tge - 1 among the first rem such.  A selected
// slot's place in the list is the count of selected slots before it: the counts of each
// (piece u, wave) go through LDS (tot: 128 ceil(NP / 8) words, free on entry), one wave scan
// over them gives each wave its offset for every u, and ballots with mbcnt give each
// lane its place within the wave.  The stores of one (u, h) are then short runs of
// consecutive places.  Returns the number selected.  Every thread must call; one
// barrier, none after (tot is left dirty).
template <int NP, int W, bool EQ>
__device__ __forceinline__ int emit_pieces_impl(const uint32_t (&kr)[NP * W], const uint32_t (&pr)[NP * W], int np,
                                                uint32_t Tge, int rem, int32_t* out, int k, uint32_t* tot,
                                                uint64_t* stp) {
  static_assert(NWAVE == 8 && NP <= 16, "a block of 64 counts holds 8 pieces of every wave");
  constexpr int QB = (NP + 7) / 8;                  // blocks of 64 (piece, wave) counts
  const int lane = lane_id(), wv = wave_id();
  const uint32_t T = Tge - 1u;
  uint32_t* const tg = tot;
  uint32_t* const te = tot + QB * 64;
  uint32_t cg_l = 0u, ce_l = 0u;
#pragma unroll
  for (int u = 0; u < NP; u++) {
    uint32_t g = 0u, e = 0u;
    if (u < np) {
#pragma unroll
      for (int h = 0; h < W; h++) {
        g += (uint32_t)__popcll(__ballot(kr[W * u + h] >= Tge));
        if (EQ) e += (uint32_t)__popcll(__ballot(kr[W * u + h] == T));
      }
    }
    cg_l = lane == u ? g : cg_l;                    // lane u writes piece u's counts
    if (EQ) ce_l = lane == u ? e : ce_l;
  }
  if (lane < NP) {
    tg[lane * NWAVE + wv] = cg_l;
    if (EQ) te[lane * NWAVE + wv] = ce_l;
  }
  __syncthreads();
  STAMPP(stp, 11);
  uint32_t og[QB], oe[QB];
  uint32_t cg = 0u, ce = 0u;
#pragma unroll
  for (int c = 0; c < QB; c++) {
    const int q = c * 64 + lane;
    const uint32_t xg = q < NP * NWAVE ? tg[q] : 0u;
    const uint32_t ig = (uint32_t)wave_incl_scan((int)xg);
    og[c] = cg + ig - xg;
    cg += rl(ig, 63);
    if (EQ) {
      const uint32_t xe = q < NP * NWAVE ? te[q] : 0u;
      const uint32_t ie = (uint32_t)wave_incl_scan((int)xe);
      oe[c] = ce + ie - xe;
      ce += rl(ie, 63);
    }
  }
  STAMPP(stp, 12);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(out, (int64_t)k * 4);
  constexpr int OOB = 0x7FFFFFF0;
#pragma unroll
  for (int u = 0; u < NP; u++) {
    if (u >= np) continue;                          // (no break: the loop must unroll, kr and pr stay in registers)
    const int ql = (u % 8) * 8 + wv;                // this wave's count of piece u in block u / 8
    int rg = (int)rl(og[u / 8], ql), re = 0;
    if (EQ) re = (int)rl(oe[u / 8], ql);
#pragma unroll
    for (int h = 0; h < W; h++) {
      const uint64_t mg = __ballot(kr[W * u + h] >= Tge);
      rg += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, 0u));
      if (EQ) {
        const uint64_t me = __ballot(kr[W * u + h] == T);
        re += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
      }
    }
#pragma unroll
    for (int h = 0; h < W; h++) {
      const uint32_t key = kr[W * u + h];
      const bool sg = key >= Tge;
      bool sel = sg;
      int o = rg;
      if (EQ) {
        const bool se = key == T;
        sel = sg || (se && re < rem);
        o = rg + (re < rem ? re : rem);
        re += se ? 1 : 0;
      }
      __builtin_amdgcn_raw_buffer_store_b32(pr[W * u + h], rout, sel ? o * 4 : OOB, 0, 0);
      rg += sg ? 1 : 0;
    }
  }
  return (int)cg + (EQ ? ((int)ce < rem ? (int)ce : rem) : 0);
}

template <int NP, int W>
__device__ __forceinline__ int emit_pieces(const uint32_t (&kr)[NP * W], const uint32_t (&pr)[NP * W], int np,
                                           uint32_t Tge, int rem, int32_t* out, int k, uint32_t* tot,
                                           uint64_t* stp = nullptr) {
  return rem > 0 ? emit_pieces_impl<NP, W, true>(kr, pr, np, Tge, rem, out, k, tot, stp)
                 : emit_pieces_impl<NP, W, false>(kr, pr, np, Tge, 0, out, k, tot, stp);
}

// Exact top-k of row scores in global memory (n > k), one workgroup, LDS for the
// histogram only.  Radix passes of 11, 11 and 10 bits over all scores (16-byte loads, 32
// keys a thread in flight) find the k-th key; they stop early once every key of the
// digit found is selected, or when all keys are equal (min = max, from the first pass).
// The result is (Tge, rem): every key >= Tge is selected, and the first rem keys equal to
// Tge - 1.  An ordered emission (16 consecutive positions a thread, one block scan a
// round) writes the list and stops once k positions are out.  Every thread must call.
__device__ __noinline__ void emit_ordered(const float* row, int n, int k, uint32_t Tge, int trem, int32_t* out,
                                          int* misc);

__device__ __noinline__ void global_select_row(const float* row, int n, int k, int32_t* out, uint32_t* hist, int* misc) {
  const int tid = threadIdx.x;
  __amdgpu_buffer_rsrc_t rs = make_rsrc(row, (int64_t)n * 4);
  constexpr int U = 8;                                // 16-byte loads a thread per round
  constexpr int ROUND = NT * 4 * U;
  uint32_t prefix = 0, mask = 0, Tge = 0;
  int rem = k, trem = 0;
  bool resolved = false;
  for (int pass = 0; pass < 3 && !resolved; pass++) {
    const int width = pass < 2 ? 11 : 10;
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = 1 << width;
    for (int b = tid; b < nb; b += NT) hist[b] = 0;
    __syncthreads();
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int base = 0; base < n; base += ROUND) {
      v4u v[U];
#pragma unroll
      for (int u = 0; u < U; u++)
        v[u] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, (base + (u * NT + tid) * 4) * 4, 0, 0));
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const int p = base + (u * NT + tid) * 4 + c;
          const bool valid = p < n;
          const uint32_t key = radix_key(__uint_as_float(v[u][c]));
          if (pass == 0) {
            mn = min(mn, valid ? key : 0xFFFFFFFFu);
            mx = max(mx, valid ? key : 0u);
          }
          hist_add(hist, valid && (key & mask) == prefix, (key >> shift) & (uint32_t)(nb - 1));
        }
    }
    if (pass == 0) {
      block_min_max(mn, mx, misc);
      if (mn == mx) {                                 // all keys equal: the first k of them
        Tge = mn + 1u;
        trem = k;
        break;
      }
    }
    __syncthreads();
    find_digit(hist, nb, rem, misc);
    const uint32_t d = (uint32_t)misc[8];
    const int r = misc[9];
    const int cnt = misc[10];
    prefix |= d << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    if (cnt == r) {                                   // every key of digit d: the keys >= prefix
      Tge = prefix;
      trem = 0;
      resolved = true;
    } else if (pass == 2) {                           // r of the keys equal to prefix
      Tge = prefix + 1u;
      trem = r;
      resolved = true;
    }
    rem = r;
    __syncthreads();
  }
  emit_ordered(row, n, k, Tge, trem, out, misc);
}

// Ordered emission over a row's scores in memory: every key >= Tge and the first trem
// keys equal to Tge - 1, in position order, into out[0 .. k); stops once k are out.
// Every thread must call.
__device__ __noinline__ void emit_ordered(const float* row, int n, int k, uint32_t Tge, int trem, int32_t* out,
                                          int* misc) {
  const int tid = threadIdx.x;
  __amdgpu_buffer_rsrc_t rs = make_rsrc(row, (int64_t)n * 4);
  const uint32_t Teq = Tge - 1u;
  int gt_carry = 0, eq_carry = 0;
  for (int base = 0; base < n; base += NT * 16) {
    const int p0 = base + tid * 16;
    uint32_t key[16];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const v4u x = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, p0 * 4 + 16 * u, 0, 0));
#pragma unroll
      for (int c = 0; c < 4; c++) key[4 * u + c] = p0 + 4 * u + c < n ? radix_key(__uint_as_float(x[c])) : 0u;
    }
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      gt += key[j] != 0u && key[j] >= Tge ? 1 : 0;
      eq += key[j] != 0u && key[j] == Teq ? 1 : 0;
    }
    int tot;
    const int packed = block_excl_scan(gt | (eq << 16), misc, &tot);
    int gtc = gt_carry + (packed & 0xFFFF), eqc = eq_carry + (packed >> 16);
#pragma unroll
    for (int j = 0; j < 16; j++) {
      if (key[j] == 0u) continue;
      if (key[j] >= Tge) {
        const int o = gtc + (eqc < trem ? eqc : trem);
        if (o < k) out[o] = p0 + j;
        gtc++;
      } else if (key[j] == Teq) {
        if (eqc < trem && gtc + eqc < k) out[gtc + eqc] = p0 + j;
        eqc++;
      }
    }
    gt_carry += tot & 0xFFFF;
    eq_carry += tot >> 16;
    if (gt_carry + (eq_carry < trem ? eq_carry : trem) >= k) break;
  }
}

// m (the rank of a chunk's local threshold: its m-th largest key), the number G of
// 32-slot groups of its candidate block and the candidate cap 32 G - 2 (slots 0 and 1
// hold the header and the maximum), from the row length n, chunk size C and k.  About
// k*C/n keys of a chunk reach the top k; m adds a margin so that the largest threshold
// over the chunks stays below the row's k-th key, and the cap leaves room for ties.
__device__ inline void candidate_params(int n, int C, int k, int* m, int* cap, int* groups) {
  // k * C <= 2^20 and n >= 1: 32-bit arithmetic is exact
  const uint32_t lam = ((uint32_t)(k * C) + (uint32_t)n - 1u) / (uint32_t)n;
  int mm = (int)(lam + lam / 4u + 12u);
  mm = mm > 64 ? 64 : mm;
  const int need = mm + (mm / 4 > 4 ? mm / 4 : 4);
  const int G = need <= 30 ? 1 : (need <= 62 ? 2 : 4);
  *m = mm;
  *cap = 32 * G - 2;
  *groups = G;
}

// A chunk's local threshold from one histogram, with no bisection: the chunk's scores
// (8 a lane, fv / their radix keys kr, 0 where no key) are counted into 128 bins linear
// in the score over [lo, largest score].  lo is the smallest lane maximum when every
// lane holds keys (the range then holds at least the 64 lane maxima, so at least m keys,
// m <= 64), else the smallest key present (every key is counted).  Bin b* is the first,
// from the top, whose running count reaches m.  The bin index is a monotone function of
// the score, so the keys of bins <= b* are exactly the keys >= the smallest of them,
// which becomes t.  Returns false (the caller bisects instead) when all keys in range
// are equal, the span is not finite, fewer than m keys are counted, or more than cap
// keys would publish and not all of them equal the chunk's maximum.
// hst: 128 words of LDS owned by this wave.  All 64 lanes must call.
__device__ __forceinline__ bool chunk_bound_linear(const float (&fv)[8], const uint32_t (&kr)[8], uint32_t lmax,
                                                   uint32_t cmax, int m, int cap, uint32_t* hst, uint32_t* t) {
  const int lane = lane_id();
  // The range starts at the smallest lane maximum when every lane holds keys (at least
  // 64 keys lie at or above it).  A lane without keys (a row's last chunk, or a chunk
  // of fewer than 512 keys, whose keys sit in the low lanes) would make that bound 0:
  // then the range starts at the smallest key present, so every key is counted.
  uint32_t lmin;
  if (__ballot(lmax == 0u) == 0ull) {
    lmin = wave_min_u32(lmax);
  } else {
    uint32_t kmn = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < 8; j++) kmn = kr[j] != 0u ? min(kmn, kr[j]) : kmn;
    lmin = wave_min_u32(kmn);
    if (lmin == 0xFFFFFFFFu) return false;          // no key at all
  }
  if (lmin == cmax) return false;
  const float hf = key_float(cmax), lf = key_float(lmin);
  const float span = hf - lf;
  const float scale = 128.0f * __builtin_amdgcn_rcpf(span);   // any positive scale keeps the bins monotone
  if (!(span <= 3.0e38f) || !(scale <= 3.0e38f)) return false;
  reinterpret_cast<uint64_t*>(hst)[lane] = 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint32_t bn[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    bn[j] = (kr[j] != 0u && fv[j] >= lf) ? min(__float2uint_rz((hf - fv[j]) * scale), 127u) : 128u;
    if (bn[j] < 128u) atomicAdd(&hst[bn[j]], 1u);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t h2 = reinterpret_cast<const uint64_t*>(hst)[lane];   // bins 2 lane, 2 lane + 1
  const int c0 = (int)(uint32_t)h2, c1 = (int)(uint32_t)(h2 >> 32);
  const int incl = wave_incl_scan(c0 + c1);                            // keys in bins <= 2 lane + 1
  const uint64_t r1 = __ballot(incl >= m);
  if (r1 == 0ull) return false;
  const int f = __ffsll((unsigned long long)r1) - 1;
  const bool first = ((__ballot(incl - c1 >= m) >> f) & 1ull) != 0ull;
  const uint32_t bstar = 2u * (uint32_t)f + (first ? 0u : 1u);
  const int count = __builtin_amdgcn_readlane(first ? incl - c1 : incl, f);
  uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < 8; j++) mn = bn[j] <= bstar ? min(mn, kr[j]) : mn;
  *t = wave_min_u32(mn);
  // past cap, a bisection may find a tighter bound, unless every key counted equals the
  // chunk's maximum (a tie at the top): then t is exact and the chunk overflows with it
  return count <= cap || *t == cmax;
}

// Whether any / every thread of the workgroup holds p (misc[48 .. 56) as scratch).
// Every thread must call; two barriers.
__device__ __forceinline__ bool block_any(bool p, int* misc) {
  const int w = __ballot(p) != 0 ? 1 : 0;
  if (lane_id() == 0) misc[48 + wave_id()] = w;
  __syncthreads();
  const v4i a = reinterpret_cast<const v4i*>(misc)[12];
  const v4i b = reinterpret_cast<const v4i*>(misc)[13];
  __syncthreads();
  return (a[0] | a[1] | a[2] | a[3] | b[0] | b[1] | b[2] | b[3]) != 0;
}

// ---------------------------------------------------------------------------
// scoring of one chunk: scores of the group's rows land in sc_lds[row][0..C)
// TS = tile stride = waves per row (8 / R, 2 for R = 3); each wave scores one row.
// ---------------------------------------------------------------------------
// Keys written in this launch that fall in the chunk: bit b of `hit` is the request's
// row b, whose key takes position readlane(npos, b) with scale readlane(nscl, b); its
// codes are at L_PATCH + 128 b.  `mine` marks the rows of this workgroup's group, whose
// keys it also stores to the cache.
struct Patches {
  uint64_t hit, mine;
  int npos;
  float nscl;
};

// The group's queries, head weights and (with PATCH) the request's new key codes, as
// 16-byte pieces in registers: thread t holds pieces t, t + NT, ... of each array.
struct Staged {
  v4u q[2 * GR];
  v4u w, codes;
};

template <int P, int TS, bool PATCH>
__device__ __forceinline__ void score_chunk(const KArgs& a, uint8_t* smem, int R, int c, const int* phys,
                                            const Patches& pt, int srec, const Staged& sg) {
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  float* const sc_lds = LDS_PTR(float, L_SC);
  constexpr int T = (2 * P + TS - 1) / TS;      // tiles of 32 keys per wave
  constexpr int KS = key_slots(P, TS);          // page slots of the LDS ring
  constexpr int LQ = l_q(P, TS);                // the queries, after the ring
  const int lr = wv / TS;                       // this wave's row (>= R: an idle wave)
  const int toff = wv % TS;
  const bool live = lr < R;
  const int lrr = live ? lr : 0;
  const int g2 = lane >> 5;

  // Key pages stream through registers: thread t loads bytes [16 t, 16 t + 16) of a page
  // (key t / 8, 16-byte chunk t % 8; one coalesced 8 KiB read a page), and threads [0, 64)
  // one key scale each.  Ordinary vector loads: the compiler counts them and waits for
  // exactly the page being staged.  Staging widens the 16 E4M3 codes to bf16 (exact: every
  // finite E4M3 value is a bf16 value) once for all the waves that read them, and writes
  // 16-byte chunk e (8 dimensions) of key kn at position e ^ (kn % 16) of the key's 256
  // bytes, so that the operand reads below (32 keys, one chunk each) hit distinct banks.
  v4u pgv[P];
  uint32_t psv[P];
  auto issue_page = [&](int j) {
    pgv[j] = *reinterpret_cast<const v4u*>(a.kc + (int64_t)phys[j] * (PS * D) + tid * 16);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.ks + (int64_t)phys[j] * PS, PS * 4);
    psv[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rk, tid < PS ? tid * 4 : 0x7FFFFFF0, 0, 0);
  };
  // 16 E4M3 codes (4 words) to 16 bf16 (two 16-byte chunks), and their place in a key row
  auto widen16 = [](const v4u x, v4u& lo, v4u& hi) {
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, false));
      const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, true));
      if (w < 2) { lo[2 * w] = p0; lo[2 * w + 1] = p1; }
      else { hi[2 * (w - 2)] = p0; hi[2 * (w - 2) + 1] = p1; }
    }
  };
  auto key_row = [&](int j, int kn) { return smem + L_KEYS + (j % KS) * PAGE16 + kn * (D * 2); };
  auto stage_page = [&](int j) {
    const int kn = tid >> 3, e = tid & 7;
    v4u lo, hi;
    widen16(pgv[j], lo, hi);
    uint8_t* kb = key_row(j, kn);
    *reinterpret_cast<v4u*>(kb + (((2 * e) ^ (kn & 15)) << 4)) = lo;
    *reinterpret_cast<v4u*>(kb + (((2 * e + 1) ^ (kn & 15)) << 4)) = hi;
    if (tid < PS) LDS_PTR(uint32_t, L_KSC)[j * PS + tid] = psv[j];
  };
  constexpr int LA = lookahead(TS);
  constexpr int L0 = (P < LA + 1) ? P : LA + 1;
#pragma unroll
  for (int j = 0; j < L0; j++) issue_page(j);
  // the queries, head weights and new key codes into LDS (their loads were issued before
  // the pages', so waiting for them leaves the pages in flight)
  {
#pragma unroll
    for (int u = 0; u < 2 * GR; u++) {
      const int off = (u * NT + tid) * 16;                 // byte offset in the group's queries
      const int rr = off >> 14, h = (off >> 8) & (H - 1), cpos = (off >> 4) & 15;
      if (u < 2 * R)
        *reinterpret_cast<v4u*>(smem + LQ + rr * (H * D * 2) + h * (D * 2) + ((cpos ^ (h & 15)) << 4)) = sg.q[u];
    }
    if (tid < R * (H * 2 / 16)) *reinterpret_cast<v4u*>(smem + L_W + tid * 16) = sg.w;
    if (PATCH && tid < NEW_MAX * (D / 16)) *reinterpret_cast<v4u*>(smem + L_PATCH + tid * 16) = sg.codes;
  }
  __syncthreads();                              // the queries and head weights are in LDS

  // A operands: bf16 MFMA 32x32x16, lane l supplies row l % 32 and 8 consecutive k of
  // its half l / 32.  K step s of half g covers d = 64 g + 8 s .. +8 (the keys use the
  // same mapping); M tile mt covers heads 32 mt .. +32.
  v8bf aq[2][8];
  float wr[2][16];
  {
    const uint8_t* qrow = smem + LQ + lrr * (H * D * 2);
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const int h = mt * 32 + (lane & 31);
#pragma unroll
      for (int st = 0; st < 8; st++) {
        const v4i x = *reinterpret_cast<const v4i*>(qrow + h * (D * 2) + (((g2 * 8 + st) ^ (h & 15)) << 4));
        aq[mt][st] = __builtin_bit_cast(v8bf, x);
      }
    }
    const uint16_t* wl = LDS_PTR(const uint16_t, L_W) + lrr * H;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int i = 0; i < 16; i++)
        wr[mt][i] = __uint_as_float(((uint32_t)wl[mt * 32 + (i >> 2) * 8 + g2 * 4 + (i & 3)]) << 16);
  }
  const float* ksl = LDS_PTR(const float, L_KSC);

  // B operand of K step st of this wave's tile i: key kn = (t & 1) * 32 + lane % 32 of
  // page t / 2 (t = toff + i TS), dimensions 64 g2 + 8 st .. + 8, in bf16
  auto load_b = [&](int i, int st) -> v8bf {
    const int t = toff + i * TS;
    const int kn = (t & 1) * 32 + (lane & 31);
    const uint8_t* kb = key_row(t >> 1, kn);
    return __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(kb + (((g2 * 8 + st) ^ (kn & 15)) << 4)));
  };
  // the head-weighted ReLU sum of one M tile's 16 accumulator rows
  auto head_sum = [&](int mt, const v16f& acc) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
      s0 = fmaf(wr[mt][q], relu(acc[q]), s0);
      s1 = fmaf(wr[mt][q + 1], relu(acc[q + 1]), s1);
    }
    return s0 + s1;
  };
  // the key scale of this lane's key in tile i (read ahead of the tile's last sums)
  auto key_scale = [&](int i) {
    const int t = toff + i * TS;
    return ksl[(t >> 1) * PS + (t & 1) * 32 + (lane & 31)];
  };
  // tile i's score: both M tiles' sums, the two lane halves (lane l < 32 takes lane l + 32's
  // sum by a permlane32 swap, a VALU lane move: no LDS round trip inside the MFMA chains),
  // then x s (canonical +0)
  auto finish = [&](int i, float part0, float part1, float ksv) {
    const int t = toff + i * TS;
    const float sum = part0 + part1;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum), false, false);
    const float tot = sum + __uint_as_float(sw[1]);
    if (live && lane < 32) sc_lds[lr * CMAX + t * 32 + lane] = tot * ksv + 0.0f;
  };
  // the highest page any wave reads at iteration i
  auto page_of_iter = [&](int i) { return ((i * TS + TS - 1) >> 1) < P - 1 ? ((i * TS + TS - 1) >> 1) : P - 1; };

  int issued = L0;
  int staged = -1;                              // pages [0, staged] are in the ring
  int patched = -1;                             // pages [0, patched] hold this launch's new keys
  const int cbase = c * (P * PS);
  // the new keys of pages (patched, x] into the staged pages (wave 0: 8 lanes of codes,
  // widened as the pages are, one lane of scale), and into the cache for this group's
  // rows; then a barrier
  auto patch_pages = [&](int x) {
    uint64_t todo = 0;
    for (uint64_t m = pt.hit; m != 0; m &= m - 1) {
      const int b = __builtin_ctzll(m);
      const int j = (__builtin_amdgcn_readlane(pt.npos, b) - cbase) >> 6;
      if (j > patched && j <= x) todo |= 1ull << b;
    }
    patched = x;
    if (todo == 0) return;
    if (wv == 0) {
      for (uint64_t m = todo; m != 0; m &= m - 1) {
        const int b = __builtin_ctzll(m);
        const int pos = __builtin_amdgcn_readlane(pt.npos, b);
        const int j = (pos - cbase) >> 6, kn = pos & (PS - 1);
        const bool store = (pt.mine >> b) & 1ull;
        const int64_t slot = (int64_t)phys[j] * PS + kn;
        if (lane < 8) {
          const v4u v = *reinterpret_cast<const v4u*>(smem + L_PATCH + b * D + lane * 16);
          v4u lo, hi;
          widen16(v, lo, hi);
          uint8_t* kb = key_row(j, kn);
          *reinterpret_cast<v4u*>(kb + (((2 * lane) ^ (kn & 15)) << 4)) = lo;
          *reinterpret_cast<v4u*>(kb + (((2 * lane + 1) ^ (kn & 15)) << 4)) = hi;
          if (store) *reinterpret_cast<v4u*>(a.kc_w + slot * D + lane * 16) = v;
        } else if (lane == 8) {
          const float sv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pt.nscl), b));
          LDS_PTR(float, L_KSC)[j * PS + kn] = sv;
          if (store) a.ks_w[slot] = sv;
        }
      }
    }
    __syncthreads();
  };
  auto ensure_page = [&](int x) {
    // pages through x + LA issued, pages [0, x] staged by every thread, a barrier
#pragma unroll
    for (int j = 0; j < P; j++)
      if (j >= issued && j <= x + LA) issue_page(j);
    if (issued < x + LA + 1) issued = (x + LA + 1 < P) ? x + LA + 1 : P;
#pragma unroll
    for (int j = 0; j < P; j++)
      if (j > staged && j <= x) stage_page(j);
    if (staged < x) staged = x;
    __syncthreads();
    if constexpr (PATCH) {
      if (pt.hit != 0ull) patch_pages(x);
    }
  };

  ensure_page(page_of_iter(0));
  STAMP(a, srec, 2);
  // B operands of the tile being computed; each K step's registers take the next tile's
  // operand once that step's second MFMA is issued.  The two M tiles run as two MFMA
  // chains, each overlapped with the other tile's head sum, so that two accumulators
  // are live at a time: chain 0 of tile i with the M tile 1 sum of tile i - 1, chain 1
  // of tile i with the M tile 0 sum of tile i.
  v8bf bq[8];
#pragma unroll
  for (int st = 0; st < 8; st++) bq[st] = load_b(0, st);
  v16f accp1 = {};
  float part0 = 0.f, kscp = 0.f;
#pragma unroll
  for (int i = 0; i < T; i++) {
    const float ksc = key_scale(i);
    // the ring slot the next tile's page takes was last read two iterations ago: this
    // barrier orders those reads before the staging writes
    if (i + 1 < T) ensure_page(page_of_iter(i + 1));
    v16f acc0 = {};
#pragma unroll
    for (int st = 0; st < 8; st++) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[0][st], bq[st], acc0, 0, 0, 0);
    if (i > 0) finish(i - 1, part0, head_sum(1, accp1), kscp);
#pragma unroll
    for (int st = 0; st < 8; st++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                             // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);                             // 5 VALU
    }
    v16f acc1 = {};
#pragma unroll
    for (int st = 0; st < 8; st++) {
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[1][st], bq[st], acc1, 0, 0, 0);
      if (i + 1 < T) bq[st] = load_b(i + 1, st);
    }
    part0 = head_sum(0, acc0);
#pragma unroll
    for (int st = 0; st < 8; st++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                             // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                             // 4 VALU
      if (i + 1 < T) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);             // 1 DS read
    }
    accp1 = acc1;
    kscp = ksc;
  }
  finish(T - 1, part0, head_sum(1, accp1), kscp);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
// t[0] and t[3] summed, t[1] and t[2] maxed over the workgroup.  Every thread must call.
__device__ __forceinline__ void block_sum_max_max_sum(uint32_t (&t)[4], int* misc) {
  const uint32_t a = wave_sum_u32(t[0]), b = wave_max_u32(t[1]), c = wave_max_u32(t[2]), d = wave_sum_u32(t[3]);
  const int wv = wave_id();
  if (lane_id() == 0) {
    misc[wv] = (int)a;
    misc[NWAVE + wv] = (int)b;
    misc[2 * NWAVE + wv] = (int)c;
    misc[3 * NWAVE + wv] = (int)d;
  }
  __syncthreads();
  uint32_t sa = 0, mb = 0, mc = 0, sd = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; i++) {
    sa += (uint32_t)misc[i];
    mb = max(mb, (uint32_t)misc[NWAVE + i]);
    mc = max(mc, (uint32_t)misc[2 * NWAVE + i]);
    sd += (uint32_t)misc[3 * NWAVE + i];
  }
  __syncthreads();
  t[0] = sa;
  t[1] = mb;
  t[2] = mc;
  t[3] = sd;
}

// The same four figures when only lanes 0, 16, 32 and 48 of each wave can hold nonzero
// values (a row's chunk headers, piece-major): readlanes instead of row reductions,
// misc[32 .. 64) as scratch.  One barrier: the caller orders any later write of
// misc[32 .. 64) behind another.  Every thread must call.
__device__ __forceinline__ void header_reduce_sparse(uint32_t (&t)[4], int* misc) {
  uint32_t v[4];
  v[0] = rl(t[0], 0) + rl(t[0], 16) + rl(t[0], 32) + rl(t[0], 48);
  v[1] = max(max(rl(t[1], 0), rl(t[1], 16)), max(rl(t[1], 32), rl(t[1], 48)));
  v[2] = max(max(rl(t[2], 0), rl(t[2], 16)), max(rl(t[2], 32), rl(t[2], 48)));
  v[3] = rl(t[3], 0) + rl(t[3], 16) + rl(t[3], 32) + rl(t[3], 48);
  v4u* const red = reinterpret_cast<v4u*>(misc + 32);
  if (lane_id() == 0) red[wave_id()] = v4u{v[0], v[1], v[2], v[3]};
  __syncthreads();
  uint32_t sa = 0, mb = 0, mc = 0, sd = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; i++) {
    const v4u x = red[i];
    sa += x[0];
    mb = max(mb, x[1]);
    mc = max(mc, x[2]);
    sd += x[3];
  }
  t[0] = sa;
  t[1] = mb;
  t[2] = mc;
  t[3] = sd;
}

// Candidate blocks: chunk w of a row owns the 32 G 8-byte slots [32 G w, 32 G w + 32 G)
// of the row's block area (G from candidate_params; the area has room for CAP_MAX slots
// a chunk), all written by every call that uses them.  Slot 0 is the header t_w |
// (overflow << 16 | count) << 32, slot 1 the chunk's largest key, slots 2 .. count + 1
// the candidates as key << 32 | position, ascending in position, and the rest zero.  The
// upper word of a header, a maximum or a zero slot is below any key, so "upper word >=
// t*" alone picks the candidates that count.

// loads a lane issues per gather batch (two slots each)
constexpr int GQ = 8;

// chunks a batch covers (all waves)
__host__ __device__ inline int batch_chunks(int G) { return NWAVE * GQ * 4 / G; }

// One batch of the gather: wave v reads, with 16-byte loads, the 32 G slots of each of
// the chunks w0 .. w0 + 4 GQ / G (w0 = b0 + v 4 GQ / G).  Load q of lane l covers slots
// 2 (l % 16 G), + 1 of chunk w0 + q 4 / G + l / 16 G, so within a wave the loads run in
// chunk order and the lanes of a load in chunk and slot order.  All loads are issued
// before any is used; chunks at or past wact point outside the buffer resource (no
// traffic, zero result).
template <int G>
__device__ __forceinline__ void gather_issue(__amdgpu_buffer_rsrc_t rent, int wact, int b0, uint64_t (&e)[2 * GQ]) {
  constexpr int OOB = 0x7FFFFFF0;
  constexpr int LPC = 16 * G;                         // lanes per chunk
  const int lane = lane_id();
  const int w0 = b0 + wave_id() * (GQ * 4 / G) + lane / LPC;
  const int slot = 2 * (lane % LPC);
#pragma unroll
  for (int q = 0; q < GQ; q++) {
    const int w = w0 + q * (4 / G);
    const int off = w < wact ? (w * 32 * G + slot) * 8 : OOB;
    const v4u x = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rent, off, 0, 0));
    e[2 * q] = ((uint64_t)x[1] << 32) | x[0];
    e[2 * q + 1] = ((uint64_t)x[3] << 32) | x[2];
  }
}

// The candidates of a loaded batch with key >= lo into cand[E0 ...], in position order
// (within a load the lanes run in slot and chunk order, two slots a lane): a ballot per
// load and slot parity ranks the kept slots within the wave, the wave totals place the
// waves.  Dropped slots write to the 64 dummy entries past FIN_ENT.  Returns the
// batch's kept count, or -1 (writing nothing) when E0 plus that count would pass
// FIN_ENT.  Every thread must call.
__device__ __forceinline__ int gather_place(const uint64_t (&e)[2 * GQ], uint32_t lo, int E0, uint64_t* cand, int* misc) {
  const int lane = lane_id(), wv = wave_id();
  int o = 0;
  int r0[GQ], r1[GQ];
#pragma unroll
  for (int q = 0; q < GQ; q++) {
    const bool k0 = (uint32_t)(e[2 * q] >> 32) >= lo;
    const bool k1 = (uint32_t)(e[2 * q + 1] >> 32) >= lo;
    const uint64_t m0 = __ballot(k0), m1 = __ballot(k1);
    const int before = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m0 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m0, 0u)) +
                       (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m1 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m1, 0u));
    r0[q] = k0 ? o + before : -1;
    r1[q] = k1 ? o + before + (k0 ? 1 : 0) : -1;
    o += (int)__popcll(m0) + (int)__popcll(m1);
  }
  if (lane == 0) misc[wv] = o;
  __syncthreads();
  const v4i ta = reinterpret_cast<const v4i*>(misc)[0];
  const v4i tb = reinterpret_cast<const v4i*>(misc)[1];
  const int t[8] = {ta[0], ta[1], ta[2], ta[3], tb[0], tb[1], tb[2], tb[3]};
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; i++) {
    before += (i < wv) ? t[i] : 0;
    tot += t[i];
  }
  __syncthreads();
  if (E0 + tot > FIN_ENT) return -1;                 // would not fit: nothing written
  const int base = E0 + before;
  const int dummy = FIN_ENT + lane;
#pragma unroll
  for (int q = 0; q < GQ; q++) {
    cand[r0[q] >= 0 ? base + r0[q] : dummy] = e[2 * q];
    cand[r1[q] >= 0 ? base + r1[q] : dummy] = e[2 * q + 1];
  }
  return tot;
}

// slots a thread holds for E entries: a multiple of 4
// The LDS slot of 16-byte piece c of an area that threads fill in one order and read in
// another: c / 8 keeps its 128-byte group, and the piece's place in the group is XORed
// with (c / 8) % 8.  A lane that reads a run of pieces, at a stride of 4 to 16 pieces
// between lanes, then meets distinct banks in eight consecutive lanes (with a plain
// layout they would all meet one bank group); consecutive pieces, as written, still fall
// in one permuted group.
__device__ __forceinline__ int swz16(int c) { return (c & ~7) | ((c ^ (c >> 3)) & 7); }

__device__ __forceinline__ int slots_for(int E) { return ((E + NT - 1) / NT + 3) & ~3; }

// zero cand[E .. NT S) (S = slots_for(E)); no barrier
__device__ __forceinline__ void pad_cand(uint64_t* cand, int E) {
  const int end = NT * slots_for(E);
  for (int e = E + (int)threadIdx.x; e < end; e += NT) cand[e] = 0ull;
}

// Top k of the E candidates cand[0 .. E) (in position order, keys within [lo, hi], zero
// up to NT slots_for(E)).  Thread t holds candidates [t S, t S + S); the candidate area
// stages the output once they are in registers.  Both histogram buffers must be clear.
// Returns false (writing nothing) when fewer than k are present.  Every thread must call.
template <int SMAX>
__device__ __forceinline__ bool select_cand(uint64_t* cand, int E, uint32_t lo, uint32_t hi, int k, uint32_t* hist,
                                            int* misc, int32_t* out, int* got, uint64_t* stp = nullptr) {
  const int S = slots_for(E);
  const v4u* src = reinterpret_cast<const v4u*>(cand + threadIdx.x * S);
  uint32_t kr[SMAX], pr[SMAX];
#pragma unroll
  for (int g = 0; g < SMAX / 4; g++) {
    if (g * 4 < S) {
      const v4u x = src[2 * g], y = src[2 * g + 1];
      pr[g * 4 + 0] = x[0]; kr[g * 4 + 0] = x[1];
      pr[g * 4 + 1] = x[2]; kr[g * 4 + 1] = x[3];
      pr[g * 4 + 2] = y[0]; kr[g * 4 + 2] = y[1];
      pr[g * 4 + 3] = y[2]; kr[g * 4 + 3] = y[3];
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) { kr[g * 4 + jj] = 0u; pr[g * 4 + jj] = 0u; }
    }
  }
  uint32_t Tge;
  int rem;
  STAMPP(stp, 5);
  if (!kth_select<SMAX>(kr, S, E, lo, hi, k, hist, misc, &Tge, &rem, stp)) return false;
  STAMPP(stp, 3);
  *got = emit_segments<SMAX>(kr, pr, S, Tge, rem, out, k, misc);
  return true;
}

// Top k of all n keys of a row held at their positions (the 16-byte piece of positions
// 4c .. 4c + 3 at piece swz16(c) of fk, zero up to NT slots_for(n)), keys within
// [lo, hi].  As select_cand otherwise (MASKED: as emit_segments).
template <int SMAX, bool MASKED>
__device__ __forceinline__ bool select_all(uint32_t* fk, int n, uint32_t lo, uint32_t hi, int k, uint32_t* hist,
                                           int* misc, int32_t* out, int* got, uint64_t* stp = nullptr) {
  const int S = slots_for(n);
  const int e0 = threadIdx.x * S;
  const v4u* src = reinterpret_cast<const v4u*>(fk);
  uint32_t kr[SMAX], pr[SMAX];
#pragma unroll
  for (int g = 0; g < SMAX / 4; g++) {
    const v4u x = g * 4 < S ? src[swz16((e0 >> 2) + g)] : v4u{0u, 0u, 0u, 0u};
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      kr[g * 4 + jj] = x[jj];
      pr[g * 4 + jj] = (uint32_t)(e0 + g * 4 + jj);
    }
  }
  uint32_t Tge;
  int rem;
  STAMPP(stp, 5);
  if (!kth_select<SMAX>(kr, S, n, lo, hi, k, hist, misc, &Tge, &rem, stp)) return false;
  STAMPP(stp, 3);
  *got = emit_segments<SMAX, MASKED>(kr, pr, S, Tge, rem, out, k, misc);
  return true;
}

// A position as a radix key that decreases with the position: the key of the finite f32
// 2^20 - pos (exact for the positions of a candidate row, which has at most 2,048 chunks
// of at most 512 keys).  kth_select over these keys picks the lowest positions.
constexpr uint32_t CAND_POS_LIMIT = 1u << 20;
__device__ __forceinline__ uint32_t pos_key(uint32_t pos) { return radix_key((float)(CAND_POS_LIMIT - pos)); }
static_assert(4 * NT * CMAX <= (int)CAND_POS_LIMIT && CAND_POS_LIMIT <= (1u << 24), "positions as exact f32");

// The list of the keys >= Tge among cand[0 .. E1), and of the keys equal to tkey whose
// position key (pos_key) is at least pcut, when cand[0 .. E0) and cand[E0 .. E1)
// each hold distinct positions in ascending order (and no position is in both): each
// run's kept positions are compacted in order into buf (wave ballots, one block scan),
// then the two sorted runs are merged, thread t writing list entries [4 t, 4 t + 4)
// from the split a binary search finds on its diagonal (merge path).  The work is
// spread over the entries however the kept ones crowd together.  buf holds k words.
// Returns the number kept.  Every thread must call.
__device__ __forceinline__ int emit_merged(const uint64_t* cand, int E0, int E1, uint32_t Tge, uint32_t tkey,
                                           uint32_t pcut, int k, uint32_t* buf, int* misc, int32_t* out) {
  constexpr int SR = FIN_ENT / NT;
  static_assert(SR * 64 * NWAVE == FIN_ENT, "the waves' ranges tile the candidate area");
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  // wave wv takes entries [wv L, wv L + L), L = 64 nj
  const int nj = __builtin_amdgcn_readfirstlane((E1 + 64 * NWAVE - 1) / (64 * NWAVE));
  const int e0 = wv * nj * 64;
  int rk[SR];
  uint32_t ps[SR];
  int cnt = 0, cntA = 0;
  // every load first (e < NWAVE nj 64 + SR 64 <= FIN_ENT stays in the candidate area;
  // entries past the wave's range or E1 are masked), then the ballots
  uint64_t cv[SR];
#pragma unroll
  for (int j = 0; j < SR; j++) cv[j] = cand[e0 + j * 64 + lane];
#pragma unroll
  for (int j = 0; j < SR; j++) {
    const int e = e0 + j * 64 + lane;
    const uint32_t key = (uint32_t)(cv[j] >> 32);
    const bool keep = (j < nj) & (e < E1) & ((key >= Tge) | ((key == tkey) & (pos_key((uint32_t)cv[j]) >= pcut)));
    const uint64_t m = __ballot(keep);
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    rk[j] = keep ? cnt + below : -1;
    ps[j] = (uint32_t)cv[j];
    cnt += (int)__popcll(m);
    cntA += (int)__popcll(m & __ballot(e < E0));
  }
  __syncthreads();                                    // misc may still be read by the caller's last step
  if (lane == 0) {
    misc[wv] = cnt;
    misc[NWAVE + wv] = cntA;
  }
  __syncthreads();
  int off = 0, tot = 0, ka = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; i++) {
    off += i < wv ? misc[i] : 0;
    tot += misc[i];
    ka += misc[NWAVE + i];
  }
  // a dropped entry writes a dummy word past the k the list takes
#pragma unroll
  for (int j = 0; j < SR; j++) buf[rk[j] >= 0 && off + rk[j] < k ? off + rk[j] : IDX_KMAX + lane] = ps[j];
  __syncthreads();
  const int kept = tot < k ? tot : k;
  const int kA = ka < kept ? ka : kept, kB = kept - kA;
  const uint32_t* A = buf;
  const uint32_t* B = buf + kA;
  const int d = min(4 * tid, kept);
  // ia = how many of the first d list entries come from A
  int lo = max(0, d - kB), hi = min(d, kA);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (A[mid] < B[d - 1 - mid]) lo = mid + 1;
    else hi = mid;
  }
  int ia = lo, ib = d - lo;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    if (d + u < kept) {
      const uint32_t va = ia < kA ? A[ia] : 0xFFFFFFFFu;
      const uint32_t vb = ib < kB ? B[ib] : 0xFFFFFFFFu;
      const bool fromA = va < vb;
      out[d + u] = (int32_t)(fromA ? va : vb);
      ia += fromA ? 1 : 0;
      ib += fromA ? 0 : 1;
    }
  }
  __syncthreads();
  return tot;
}

// The (ceil(k / m) + 1)-th largest local threshold t_w among a row's chunks that did not
// overflow (bm[w] for w < wact; 0xFFFFFFFF marks an overflowed chunk), or *ok = false when
// fewer chunks have one.  Every thread must call.
__device__ __noinline__ uint32_t header_floor(const uint32_t* bm, int wact, int k, int m, uint32_t* hist, int* misc,
                                              bool* ok) {
  const int tid = threadIdx.x;
  uint32_t kr[4];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int w = tid + NT * u;                       // wact <= 4 NT
    const uint32_t b = w < wact ? bm[w] : 0xFFFFFFFFu;
    kr[u] = b == 0xFFFFFFFFu ? 0u : b;
    mn = min(mn, kr[u] != 0u ? kr[u] : 0xFFFFFFFFu);
    mx = max(mx, kr[u]);
  }
  block_min_max(mn, mx, misc);
  clear_hist(hist);
  __syncthreads();
  uint32_t T = 0u;
  int rem = 0;
  const int kk = (k + m - 1) / m + 1;
  *ok = mx != 0u && kth_select<4>(kr, 4, -1, mn, mx, kk, hist, misc, &T, &rem);
  return rem > 0 ? T - 1u : T;
}

// Candidate path when the certificate fails.  cand[0 .. E) holds every published key >=
// lo (chunk w published its keys >= bm[w]; bm[w] = 0xFFFFFFFF marks an overflowed chunk,
// which published none), so chunk w holds its keys >= held(w) = max(bm[w], lo).  T0 =
// the k-th candidate (if there are k), at most the row's k-th key; every chunk whose
// held range does not reach down to T0 is re-read from the row's scores for its keys in
// [T0, held(w)), after which every key >= T0 of the row is a candidate, and the top k is
// taken from that set by merging the two position-ordered runs (emit_merged); a tie cut
// at the k-th key keeps the lowest positions, found by a selection over the ties'
// position keys.
// Returns true when it selected, false to fall back to the multi-pass select over
// memory.  Every thread must call.
__device__ __noinline__ bool rare_select(uint8_t* ws, int nr, int k, int wact, int E, int C, uint32_t lo,
                                            const float* srow, uint64_t* cand, uint32_t* bm,
                                            uint32_t* hist, int* misc, int32_t* out) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(srow, (int64_t)nr * 4);
  constexpr int SR = FIN_ENT / NT;
  uint32_t kr[SR];
  // the keys into registers, and their range: lo is only a floor (the smallest finite
  // score's key when every published key is taken), and the linear pass of kth_select
  // resolves only over a range close to that of the keys
  uint32_t kmn, kmx;
  auto load_keys = [&](int n_ent) {
    const int S = slots_for(n_ent);
    kmn = 0xFFFFFFFFu;
    kmx = 0u;
    uint64_t cv[SR];
#pragma unroll
    for (int j = 0; j < SR; j++) cv[j] = cand[j * NT + tid];   // within the candidate area
#pragma unroll
    for (int j = 0; j < SR; j++) {
      // kth_select takes the keys in any arrangement: slot j of thread t is entry j NT + t
      kr[j] = j < S ? (uint32_t)(cv[j] >> 32) : 0u;
      kmn = min(kmn, kr[j] != 0u ? kr[j] : 0xFFFFFFFFu);
      kmx = max(kmx, kr[j]);
    }
    block_min_max(kmn, kmx, misc);
    return S;
  };
  uint32_t T = 0;
  int rem = 0;
  pad_cand(cand, E);
  clear_hist(hist);
  __syncthreads();
  const int S0 = load_keys(E);
  const bool full = E >= k && kth_select<SR>(kr, S0, E, kmn, kmx, k, hist, misc, &T, &rem);
  // the k-th largest candidate is Tge - 1 when ties are cut, else at least Tge
  const uint32_t lowT = full ? (rem > 0 ? T - 1u : T) : 0u;
  if (full) {
    // only the candidates >= lowT can be selected: keep them, in place and in position
    // order (thread t compacts its run [t S0, t S0 + S0); every run is read before the
    // scan's barrier, and an entry only moves down), to make room for the re-read
    uint64_t cv[SR];
    const int b0 = tid * S0;
    int c = 0;
#pragma unroll
    for (int j = 0; j < SR; j++) {
      const bool in = j < S0 && b0 + j < E;
      cv[j] = in ? cand[b0 + j] : 0ull;
      c += (in && (uint32_t)(cv[j] >> 32) >= lowT) ? 1 : 0;
    }
    int tot;
    int o = block_excl_scan(c, misc, &tot);
#pragma unroll
    for (int j = 0; j < SR; j++)
      if (j < S0 && b0 + j < E && (uint32_t)(cv[j] >> 32) >= lowT) cand[o++] = cv[j];
    E = tot;
    __syncthreads();
  }
  // failing chunks listed in bm[4 NT ...] (the thresholds occupy bm[0 .. 4 NT))
  auto held = [&](uint32_t w) {
    const uint32_t b = bm[w];
    return b == 0xFFFFFFFFu ? b : (b > lo ? b : lo);
  };
  uint32_t* fl = bm + 4 * NT;
  int nfail = 0;
  for (int w0 = 0; w0 < wact; w0 += NT) {
    const int w = w0 + tid;
    const bool f = w < wact && (!full || held((uint32_t)w) > lowT);
    int tot;
    const int o = block_excl_scan(f ? 1 : 0, misc, &tot);
    if (f) fl[nfail + o] = (uint32_t)w;
    nfail += tot;
  }
  __syncthreads();
  // the failing chunks' keys in [lowT, held(w)), in one pass over all of them: 8
  // consecutive keys a thread a round (a chunk holds a multiple of 8), appended in
  // thread order, so that cand[E .. Ecur) is in position order as cand[0 .. E) is.
  // Give up once they overflow the candidate area, or at once without a T0 (every key
  // of every chunk would be taken) when the chunks hold too many keys.
  if (!full && E + nfail * C > FIN_ENT) return false;
  const int cshift = 31 - __clz(C);
  const int tot_keys = nfail * C;
  int Ecur = E;
#pragma unroll 1
  for (int base = 0; base < tot_keys; base += NT * 8) {
    uint32_t raw[8];
    int pos[8];
    const int f0 = base + tid * 8;
    const int p0 = f0 < tot_keys ? ((int)fl[f0 >> cshift] << cshift) + (f0 & (C - 1)) : nr;
    if (p0 + 8 <= nr) {
      const v4u x = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, p0 * 4, 0, 0));
      const v4u y = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, p0 * 4 + 16, 0, 0));
#pragma unroll
      for (int j = 0; j < 4; j++) {
        raw[j] = x[j];
        raw[4 + j] = y[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; j++)
        raw[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, p0 + j < nr ? (p0 + j) * 4 : 0x7FFFFFF0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; j++) pos[j] = p0 + j;
    uint32_t key[8];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      key[j] = radix_key(__uint_as_float(raw[j]));
      const bool take = pos[j] < nr && key[j] >= lowT && key[j] < held((uint32_t)(pos[j] >> cshift));
      if (!take) pos[j] = -1;
      cnt += take ? 1 : 0;
    }
    int tot;
    int o = Ecur + block_excl_scan(cnt, misc, &tot);
    if (Ecur + tot > FIN_ENT) return false;
#pragma unroll
    for (int j = 0; j < 8; j++)
      if (pos[j] >= 0) cand[o++] = ((uint64_t)key[j] << 32) | (uint32_t)pos[j];
    Ecur += tot;
  }
  if (Ecur < k) return false;
  pad_cand(cand, Ecur);
  clear_hist(hist);
  __syncthreads();
  const int S1 = load_keys(Ecur);
  if (!kth_select<SR>(kr, S1, Ecur, kmn, kmx, k, hist, misc, &T, &rem)) return false;
  // the list is the keys >= T and the first rem keys equal to T - 1 in position order:
  // those are the rem largest position keys among the keys equal to T - 1 (positions are
  // distinct), found by one more kth_select, and a merge of the two runs emits the list
  uint32_t tkey = 0u, pcut = 0xFFFFFFFFu;
  if (rem > 0) {
    tkey = T - 1u;
    uint32_t pmn = 0xFFFFFFFFu, pmx = 0u;
#pragma unroll
    for (int j = 0; j < SR; j++) {
      const uint64_t c = cand[j * NT + tid];
      const bool tie = j < S1 && (uint32_t)(c >> 32) == tkey;
      kr[j] = tie ? pos_key((uint32_t)c) : 0u;
      pmn = min(pmn, tie ? kr[j] : 0xFFFFFFFFu);
      pmx = max(pmx, kr[j]);
    }
    block_min_max(pmn, pmx, misc);
    clear_hist(hist);
    __syncthreads();
    uint32_t Tp;
    int rp;
    if (!kth_select<SR>(kr, S1, -1, pmn, pmx, rem, hist, misc, &Tp, &rp)) return false;
    pcut = rp > 0 ? Tp - 1u : Tp;
  }
  const int got = emit_merged(cand, E, Ecur, T, tkey, pcut, k, bm, misc, out);
  if (got != k && tid == 0) raise_error(ws, IDX_DERR_SELECT);
  return true;
}

// The fast path's fallback when the chunks holding the row's top keys publish too few of
// them (the certificate failed: fewer than k keys reach t*).  The candidate set is every
// key of the J chunks with the highest thresholds t_w (the overflowed chunks first, J as
// many as the candidate area holds) and the published keys of every other chunk, placed in
// position order.  A chunk w outside the set hides only keys below t_w, so the set's top k
// is the row's when its k-th key is at least Y, the largest t_w left out; keys below Y
// count as absent.  Returns false, with nothing written to out, when the set does not fit
// or falls short of that.  On entry bm[w] holds t_w (all ones for an overflowed chunk)
// and bm[6 NT + w] the upper word of chunk w's header; bm[0 .. 4 NT) is left as it was,
// while the candidate area, both histograms and bm[4 NT .. 6 NT) are overwritten.
// wact <= NT.  Every thread must call.
__device__ __noinline__ bool select_hot_chunks(uint8_t* ws, int nr, int k, int wact, int C, int SL,
                                               const uint64_t* erow, const float* srow,
                                               uint64_t* cand, uint32_t* bm, uint32_t* hist, int* misc,
                                               int32_t* out) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rent = make_rsrc(erow, (int64_t)wact * SL * 8);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(srow, (int64_t)nr * 4);
  constexpr int SR = FIN_ENT / NT;
  constexpr int OOB = 0x7FFFFFF0;
  const int cshift = 31 - __clz(C);
  const int sshift = 31 - __clz(SL);
  // thread w < wact: chunk w's threshold and header flags
  const bool act = tid < wact;
  const uint32_t tw = act ? bm[tid] : 0u;
  const uint32_t hf = act ? bm[6 * NT + tid] : 0u;
  const bool ov = act && ((hf >> 16) & 1u);
  const uint32_t cnt = act && !ov ? (hf & 0xFFFFu) : 0u;
  const int cw_all = act ? min(C, nr - (tid << cshift)) : 0;
  uint32_t t4[4] = {ov ? 1u : 0u, 0u, 0u, cnt};
  block_sum_max_max_sum(t4, misc);
  const int n_ov = (int)t4[0], e_pub = (int)t4[3];
  const int J = min(wact, (FIN_ENT - e_pub) / C);
  if (J < n_ov) return false;
  // X: the (J - n_ov)-th largest threshold of the chunks that did not overflow (all of
  // them when J covers them; none when J = n_ov)
  const int jn = J - n_ov, n_kept = wact - n_ov;
  uint32_t X = 0xFFFFFFFFu;                          // above every key
  if (jn >= n_kept) {
    X = 0u;
  } else if (jn > 0) {
    uint32_t kr4[4] = {act && !ov ? tw : 0u, 0u, 0u, 0u};
    uint32_t mn = kr4[0] != 0u ? kr4[0] : 0xFFFFFFFFu, mx = kr4[0];
    block_min_max(mn, mx, misc);
    clear_hist(hist);
    __syncthreads();
    uint32_t T;
    int rem;
    if (!kth_select<4>(kr4, 4, -1, mn, mx, jn, hist, misc, &T, &rem)) return false;
    X = rem > 0 ? T - 1u : T;
  }
  const bool inF = act && (ov || tw >= X);
  const int cw = inF ? cw_all : (int)cnt;
  uint32_t t5[4] = {inF ? 1u : 0u, act && !inF && !ov ? tw : 0u, 0u, 0u};
  int E;
  const int off = block_excl_scan(cw, misc, &E);
  int nF;
  const int fr = block_excl_scan(inF ? 1 : 0, misc, &nF);
  block_sum_max_max_sum(t5, misc);
  const uint32_t Y = t5[1];                          // the largest threshold left out (0: none)
  if (E > FIN_ENT || (nF << cshift) > FIN_ENT) return false;
  // per chunk: its first entry and whether all its keys are taken, its published count,
  // and the list of chunks taken whole
  uint32_t* meta = bm + 4 * NT;
  uint32_t* flist = bm + 5 * NT;
  if (act) {
    meta[tid] = (uint32_t)off | (inF ? 0x80000000u : 0u);
    hist[tid] = cnt;
    if (inF) flist[fr] = (uint32_t)tid;
  }
  __syncthreads();
  // All loads first, one round trip: the blocks' slot pairs u NT + t (slot j >= 2 of
  // chunk w is its published entry j - 2), and 4 consecutive keys a thread a round of the
  // chunks taken whole.  A group that runs past the row (its last, when nr % 4 != 0) is
  // read from nr - 4 and shifted into place (nr > ALL_MAX here); groups past the chunks
  // read from outside the resource.
  constexpr int RW = FIN_ENT / (4 * NT);
  v4u pv[8];
#pragma unroll
  for (int u = 0; u < 8; u++)
    pv[u] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rent, (u * NT + tid) * 16, 0, 0));
  const int whole = nF << cshift;
  v4u kv[RW];
  int kp[RW], ksh[RW];
#pragma unroll
  for (int r = 0; r < RW; r++) {
    const int i = (r * NT + tid) * 4;
    const int w = i < whole ? (int)flist[i >> cshift] : 0;
    const int p = i < whole ? (w << cshift) + (i & (C - 1)) : nr;
    const int at = p < nr ? min(p, nr - 4) : -1;
    kp[r] = p;
    ksh[r] = p - at;
    kv[r] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, at >= 0 ? at * 4 : OOB, 0, 0));
  }
#pragma unroll
  for (int u = 0; u < 8; u++)
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++) {
      const int sl = 2 * (u * NT + tid) + h2;
      const int w = sl >> sshift, j = sl & (SL - 1);
      const bool in = w < wact;
      const uint32_t m = in ? meta[w] : 0x80000000u;
      if (!(m >> 31) && j >= 2 && j - 2 < (int)hist[in ? w : 0])
        cand[(m & 0x7FFFFFFFu) + j - 2] = ((uint64_t)pv[u][2 * h2 + 1] << 32) | pv[u][2 * h2];
    }
#pragma unroll
  for (int r = 0; r < RW; r++) {
    const int p = kp[r], sh = ksh[r];
    if (p < nr) {
      const int w = p >> cshift;
      const int base = (int)(meta[w] & 0x7FFFFFFFu) + (p & (C - 1));
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint32_t x = q + sh == 0 ? kv[r][0] : (q + sh == 1 ? kv[r][1] : (q + sh == 2 ? kv[r][2] : kv[r][3]));
        if (p + q < nr) cand[base + q] = ((uint64_t)radix_key(__uint_as_float(x)) << 32) | (uint32_t)(p + q);
      }
    }
  }
  pad_cand(cand, E);
  __syncthreads();
  // the top k of the set, keys below Y absent
  const int S = slots_for(E);
  const v4u* src = reinterpret_cast<const v4u*>(cand + tid * S);
  uint32_t kr[SR], pr[SR];
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
  for (int g = 0; g < SR / 4; g++) {
    if (g * 4 < S) {
      const v4u x = src[2 * g], y = src[2 * g + 1];
      pr[g * 4 + 0] = x[0]; kr[g * 4 + 0] = x[1];
      pr[g * 4 + 1] = x[2]; kr[g * 4 + 1] = x[3];
      pr[g * 4 + 2] = y[0]; kr[g * 4 + 2] = y[1];
      pr[g * 4 + 3] = y[2]; kr[g * 4 + 3] = y[3];
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) { kr[g * 4 + jj] = 0u; pr[g * 4 + jj] = 0u; }
    }
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      kr[g * 4 + jj] = kr[g * 4 + jj] >= Y ? kr[g * 4 + jj] : 0u;
      kmn = min(kmn, kr[g * 4 + jj] != 0u ? kr[g * 4 + jj] : 0xFFFFFFFFu);
      kmx = max(kmx, kr[g * 4 + jj]);
    }
  }
  block_min_max(kmn, kmx, misc);
  if (kmx == 0u) return false;
  clear_hist(hist);
  __syncthreads();
  uint32_t Tge;
  int rem;
  if (!kth_select<SR>(kr, S, -1, kmn, kmx, k, hist, misc, &Tge, &rem)) return false;
  // the k-th key is Tge - 1 when ties are cut, else at least Tge: every key left out must
  // lie below it (they lie below Y)
  if (Y > (rem > 0 ? Tge - 1u : Tge)) return false;
  const int got = emit_segments<SR>(kr, pr, S, Tge, rem, out, k, misc);
  if (got != k && tid == 0) raise_error(ws, IDX_DERR_SELECT);
  return true;
}

// How a row of n keys selects (the same decision in both launches): nothing to select
// (n <= k), from all its scores at once (n <= ALL_MAX), from the candidates its chunks of
// 2^shift keys publish (at most 4 NT chunks), or by a multi-pass select over its scores.
constexpr int PATH_NONE = 0, PATH_ALL = 1, PATH_CAND = 2, PATH_MULTI = 3;
__host__ __device__ inline int row_path(int n, int k, int shift) {
  if (n <= k) return PATH_NONE;
  if (n <= ALL_MAX) return PATH_ALL;
  return ((n - 1) >> shift) < 4 * NT ? PATH_CAND : PATH_MULTI;
}

// ---------------------------------------------------------------------------
// Launch 1: workgroup (c, g) scores chunk c (keys [c C, c C + C)) of request g's rows
// and, per row that selects from candidates, publishes the chunk's candidates.
// ---------------------------------------------------------------------------
// PATCH: keys written in this launch (idx_score_topk_append) are patched in; a separate
// instantiation, so that other calls carry none of it.
template <int P, bool PATCH>
__global__ __launch_bounds__(NT, 1) void score_kernel(const KArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int c = blockIdx.x;
  const int g = blockIdx.y;
  const int srec = g * gridDim.x + c;
  STAMP(a, srec, 0);
  const uint32_t ge = a.grp[g];
  const int row0 = (int)(ge & 0xFFFFFFu);
  const int R = (int)(ge >> 24);
  const int C = a.chunk;
  const int chunk_base = c * C;
  uint8_t* const ws = a.ws;
  const int gbound = a.gmax[g];
  scalars_ready(ge, gbound, a.mode, a.chunk, a.chunk_shift, a.ws, a.nk, a.pt, a.q, a.w, a.kc, a.ks, a.scores, a.ld,
                a.max_pages, a.num_pages, a.k, a.ent_stride, a.off_ent);
  if (c > 0 && chunk_base >= gbound) return;      // beyond every row of this group
  const bool do_score = (a.mode & MODE_SCORE) != 0;
  const bool do_pub = (a.mode & MODE_PUBLISH) != 0;
  // keys written in this launch: their positions and scales load with the key counts
  // below (lanes [0, request rows)), their codes with the queries
  const uint32_t rq = PATCH ? a.req[g] : 0u;
  const int rq0 = (int)(rq & 0xFFFFFFu), rqn = (int)(rq >> 24);
  int ld_np = -1, ld_rn = 0;
  float ld_ns = 0.f;
  if (do_score && lane < rqn) {
    ld_np = a.nw_pos[rq0 + lane];
    ld_ns = a.nw_scales[rq0 + lane];
    ld_rn = a.nk[rq0 + lane];                     // every request row's key count, for the position check
  }
  // n_keys of the group's rows, the chunk's page ids of every row and the workspace's
  // magic word, in one load (lanes [0, R): n_keys; lanes [8, 8 + R*P):
  // page_table[row][c*P + j]; lane 63: the magic word)
  // (three loads into distinct registers, so that none waits for another)
  int ld_nk = 0, ld_pt = 0, ld_mg = 0;
  if (lane < R) ld_nk = a.nk[row0 + lane];
  if (do_score && lane >= 8 && lane < 8 + R * P) {
    const int i = (lane - 8) / P, j = (lane - 8) % P;
    if (c * P + j < a.max_pages) ld_pt = a.pt[(int64_t)(row0 + i) * a.max_pages + c * P + j];
  }
  if (lane == 63) ld_mg = *reinterpret_cast<const int*>(ws + WS_MAGIC_OFF);
  // The group's queries (R rows of 16 KiB), head weights and the request's new key codes
  // into registers, issued after the loads above so that their wait covers only those:
  // the page loads need the page ids, not the queries.  Pieces outside each array's range
  // read zeros from outside the buffer resource (no memory traffic).
  __builtin_amdgcn_sched_barrier(0);
  Staged sg;
  if (do_score) {
    const __amdgpu_buffer_rsrc_t rq_ = make_rsrc(a.q + (int64_t)row0 * (H * D * 2), (int64_t)R * (H * D * 2));
#pragma unroll
    for (int u = 0; u < 2 * GR; u++)
      sg.q[u] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rq_, (u * NT + tid) * 16, 0, 0));
    const __amdgpu_buffer_rsrc_t rw_ = make_rsrc(a.w + (int64_t)row0 * (H * 2), (int64_t)R * (H * 2));
    sg.w = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rw_, tid * 16, 0, 0));
    if (PATCH) {
      const __amdgpu_buffer_rsrc_t rc_ = make_rsrc(a.nw_codes + (int64_t)rq0 * D, (int64_t)rqn * D);
      sg.codes = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rc_, tid * 16, 0, 0));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int ld_lane = ld_nk | ld_pt | ld_mg;   // disjoint lanes
  if (!(a.mode & MODE_NOMAGIC) && (uint32_t)__builtin_amdgcn_readlane(ld_lane, 63) != WS_MAGIC) {
    if (tid == 0 && c == 0 && g == 0) raise_error(ws, IDX_DERR_WS);
    return;
  }
  STAMP(a, srec, 1);

  int n[GR];
  int nmax = 0, rmax = 0;
  uint32_t err = 0;
#pragma unroll
  for (int i = 0; i < GR; i++) {
    int v = 0;
    if (i < R) {
      v = __builtin_amdgcn_readlane(ld_lane, i);
      if (v < 0 || v > gbound) {
        err |= IDX_DERR_NKEYS;
        v = v < 0 ? 0 : gbound;
      }
    }
    n[i] = v;
    if (v > nmax) { nmax = v; rmax = i; }
  }
  if (err && tid == 0) raise_error(ws, err);
  if (chunk_base >= nmax) return;                 // nothing of this group here
  const int k = a.k;
  const int shift = a.chunk_shift;
  if (!do_score) {
    // over given scores, only rows selecting from candidates need this chunk
    bool needed = false;
#pragma unroll
    for (int i = 0; i < GR; i++) needed |= (i < R) && chunk_base < n[i] && row_path(n[i], k, shift) == PATH_CAND;
    if (!needed) return;
  }

  float* const sc_lds = LDS_PTR(float, L_SC);
  uint64_t* const ent = reinterpret_cast<uint64_t*>(ws + a.off_ent);

  if (do_score) {
    int phys[P];
    uint32_t perr = 0;
#pragma unroll
    for (int j = 0; j < P; j++) {
      int ph = __builtin_amdgcn_readlane(ld_lane, 8 + rmax * P + j);
      if ((c * P + j) * PS < nmax) {
        if (ph < 0 || ph >= a.num_pages) { perr = IDX_DERR_PAGE; ph = 0; }
      } else {
        ph = (j == 0) ? 0 : phys[0];
      }
      phys[j] = ph;
    }
    if (perr && tid == 0) raise_error(ws, perr);
    // the request's new keys in this chunk; a position outside [-1, the row's key
    // count) is reported and ignored (each row's key is within what the row sees).
    // Every row group of the request takes the same decision: it checks each request
    // row's position against that row's own key count, clamped to the request's bound
    // as the row's own group clamps it.
    Patches pt = {0ull, 0ull, ld_np, ld_ns};
    if (PATCH && rqn > 0) {
      const int own = lane - (row0 - rq0);           // this lane's row within the group
      const int nrow = ld_rn < 0 ? 0 : (ld_rn > gbound ? gbound : ld_rn);
      const bool inr = lane < rqn;
      const bool bad = inr && (ld_np < -1 || ld_np >= nrow);
      if (__ballot(bad) != 0ull && tid == 0) raise_error(ws, IDX_DERR_NKEYS);
      pt.hit = __ballot(inr && !bad && ld_np >= chunk_base && ld_np < chunk_base + C && ld_np < nmax);
      pt.mine = __ballot(inr && own >= 0 && own < R);
    }
    if (R == 1) score_chunk<P, 8, PATCH>(a, smem, R, c, phys, pt, srec, sg);
    else if (R == 2) score_chunk<P, 4, PATCH>(a, smem, R, c, phys, pt, srec, sg);
    else score_chunk<P, 2, PATCH>(a, smem, R, c, phys, pt, srec, sg);
    STAMP(a, srec, 3);
  } else {
#pragma unroll
    for (int i = 0; i < GR; i++) {
      if (i >= R) break;
      const int nv = n[i] - chunk_base;
      const float* src = a.scores + (int64_t)(row0 + i) * a.ld + chunk_base;
      for (int p = tid; p < C; p += NT) sc_lds[i * CMAX + p] = (p < nv) ? src[p] : 0.f;
    }
    __syncthreads();
  }

  // ---------------- scores out (first: their latency overlaps the publication) ------
  // thread t stores 4 consecutive scores: row 4 t / C, positions 4 t % C .. + 4
  if (do_score && 4 * tid < R * C) {
    const int i = (4 * tid) >> a.chunk_shift, p = (4 * tid) & (C - 1);
    const int nv = n[i] - chunk_base;
    float* dst = a.scores + (int64_t)(row0 + i) * a.ld + chunk_base + p;
    const v4f v = *reinterpret_cast<const v4f*>(sc_lds + i * CMAX + p);
    if (p + 4 <= nv && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      *reinterpret_cast<v4f*>(dst) = v;
    } else {
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (p + j < nv) dst[j] = v[j];
    }
  }

  STAMP(a, srec, 4);
  // ---------------- publish (wave i handles row i) -----------------------------------
  if (do_pub && wv < R) {
    const int i = wv;
    const int nr = n[i];
    const int nv = nr - chunk_base;
    if (nv > 0 && row_path(nr, k, shift) == PATH_CAND) {
      // the chunk's candidate block (32 G slots, stored from registers):
      // slot 0 = t_w | (overflow << 16 | count) << 32 (count = the keys >= t_w, published
      // or not), slot 1 = the chunk's largest key,
      // slots 2 .. count + 1 = every key of the chunk >= t_w as key << 32 | position,
      // ascending in position, then zeros.  t_w is a lower bound of the chunk's m-th
      // largest key, so at least m keys are published.  thr0, a bound of the m-th largest
      // of the 64 lane maxima (8 keys a lane, 12 bisection steps), is one; the keys >= thr0
      // (at most 64 of them, else thr0 is t_w) are narrowed to t_w by 8 more steps over
      // [thr0, chunk max].  A chunk with more than cap keys >= t_w publishes none of them
      // and sets the overflow flag.
      const int grow = row0 + i;
      int m, cap, G;
      candidate_params(nr, C, k, &m, &cap, &G);
      const v4f* src = reinterpret_cast<const v4f*>(sc_lds + i * CMAX + lane * 8);
      const v4f f0 = src[0], f1 = src[1];
      const float fv[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
      uint32_t key[8];
      uint32_t lmax = 0;
      const int lim = nv < C ? nv : C;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        // branch-free: the key, masked off past the chunk's keys
        key[j] = radix_key(fv[j]) & (lane * 8 + j < lim ? 0xFFFFFFFFu : 0u);
        lmax = lmax > key[j] ? lmax : key[j];
      }
      const uint32_t cmax = wave_max_u32(lmax);
      uint32_t thr;
      if (!chunk_bound_linear(fv, key, lmax, cmax, m, cap, LDS_PTR(uint32_t, L_PHIST) + i * 128, &thr)) {
        const uint32_t thr0 = wave_kth_bound(lmax, m, wave_min_u32(lmax), cmax, 12);
        int cnt0 = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) cnt0 += (key[j] != 0u && key[j] >= thr0) ? 1 : 0;
        const int incl0 = wave_incl_scan(cnt0);
        const int total0 = __builtin_amdgcn_readlane(incl0, 63);
        thr = thr0;
        if (total0 <= 64) {
          uint32_t* kst = LDS_PTR(uint32_t, L_KST) + i * 64;
          int o = incl0 - cnt0;
#pragma unroll
          for (int j = 0; j < 8; j++)
            if (key[j] != 0u && key[j] >= thr0) {
              kst[o] = key[j];
              o++;
            }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const uint32_t v = lane < total0 ? kst[lane] : 0u;
          thr = wave_kth_bound(v, m, thr0, cmax, 8);
        }
      }
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < 8; j++) cnt += (key[j] != 0u && key[j] >= thr) ? 1 : 0;
      const int incl = wave_incl_scan(cnt);
      const int total = __builtin_amdgcn_readlane(incl, 63);
      const int SL = 32 * G;
      const bool fits = total <= cap;
      // Straight to the block, branch-free (a store that has no slot goes outside the
      // buffer resource and is dropped): the candidates to slots 2 .. total + 1 in position
      // order, then the header, the maximum and zeros over every other slot.
      uint64_t* blk = ent + (int64_t)grow * a.ent_stride * CAP_MAX + (int64_t)c * SL;
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(blk, (int64_t)SL * 8);
      constexpr int OOB = 0x7FFFFFF0;
      int o = 2 + incl - cnt;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const bool sel = fits && key[j] != 0u && key[j] >= thr;
        const uint64_t word = ((uint64_t)key[j] << 32) | (uint32_t)(chunk_base + lane * 8 + j);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u_t, word), rb, sel ? o * 8 : OOB, 0, 0);
        o += sel ? 1 : 0;
      }
      const int used = fits ? total + 2 : 2;
      const uint64_t head = ((uint64_t)((fits ? 0u : (1u << 16)) | (uint32_t)total) << 32) | thr;
      for (int q = lane; q < SL; q += 64) {
        const uint64_t v = q == 0 ? head : (q == 1 ? (uint64_t)cmax : 0ull);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u_t, v), rb, (q < 2 || q >= used) ? q * 8 : OOB, 0, 0);
      }
    }
  }
  STAMP(a, srec, 5);
}

// ---------------------------------------------------------------------------
// Launch 2: workgroup (i, g) selects row i of request g.  Launch 1 has ended, so its
// scores and candidates are in memory.
// ---------------------------------------------------------------------------
template <bool SHORT>
__device__ __forceinline__ bool select_row(const KArgs& a, uint8_t* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const uint32_t ge = a.grp[blockIdx.y];
  scalars_ready(ge, a.gmax[blockIdx.y], a.ws, a.nk, a.k, a.chunk, a.chunk_shift, a.topk, a.scores, a.ld,
                a.ent_stride, a.off_ent, a.mode);
  const int R = (int)(ge >> 24);
  const int i = blockIdx.x;
  const int grow = (int)(ge & 0xFFFFFFu) + (i < R ? i : R - 1);   // a row of the group either way
  const int qrec = STAMP_SELECT + blockIdx.y * 4 + i;
  STAMP(a, qrec, 0);
#ifdef IDX_STAMPS
  uint64_t* const stp = reinterpret_cast<uint64_t*>(a.ws + a.off_stamps) + (uint64_t)qrec * STAMP_SLOTS;
#else
  uint64_t* const stp = nullptr;
#endif
  uint8_t* const ws = a.ws;
  // the magic word and the row's key count in flight together, before any branch
  const uint32_t magic = *reinterpret_cast<const uint32_t*>(ws + WS_MAGIC_OFF);
  int nr = __builtin_amdgcn_readfirstlane(a.nk[grow]);
  asm volatile("" ::"s"(magic), "s"(nr));          // both loads issued before the branches below
  if (i >= R) return false;
  if (!(a.mode & MODE_NOMAGIC) && magic != WS_MAGIC) {
    if (tid == 0 && i == 0 && blockIdx.y == 0) raise_error(ws, IDX_DERR_WS);
    return false;
  }
  const int gbound = a.gmax[blockIdx.y];
  if (nr < 0 || nr > gbound) {
    if (tid == 0) raise_error(ws, IDX_DERR_NKEYS);
    nr = nr < 0 ? 0 : gbound;
  }
  const int k = a.k, C = a.chunk;
  int32_t* out = a.topk + (int64_t)grow * k;
  const int path = row_path(nr, k, a.chunk_shift);
  if (path == PATH_NONE) {
    for (int p = tid; p < k; p += NT) out[p] = p < nr ? p : -1;
    return true;
  }
  int* misc = LDS_PTR(int, L_MISC);
  uint32_t* hist = LDS_PTR(uint32_t, L_HIST);
  uint64_t* cand = LDS_PTR(uint64_t, L_CAND);
  uint32_t* bm = LDS_PTR(uint32_t, L_BM);
  const float* srow = a.scores + (int64_t)grow * a.ld;
  __amdgpu_buffer_rsrc_t rs = make_rsrc(srow, (int64_t)nr * 4);
  clear_hist(hist);                                  // ordered before use by the barriers below
  bool done = false;
  if (path == PATH_ALL) {
    // every key of the row into LDS at its position, 16-byte loads: thread t reads
    // positions 4 t + 4 NT j .. + 4; positions past the row read 0 from outside the
    // buffer resource and are stored as absent keys up to NT slots_for(nr)
    uint32_t* fk = reinterpret_cast<uint32_t*>(cand);
    constexpr int JA = ALL_MAX / (4 * NT);
    const int J = (nr + 4 * NT - 1) / (4 * NT);
    v4u kv[JA];
#pragma unroll
    for (int j = 0; j < JA; j++)
      kv[j] = j < J ? __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, j * NT * 16, 0))
                    : v4u{0u, 0u, 0u, 0u};
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;              // key - 1 domain for the minimum
#pragma unroll
    for (int j = 0; j < JA; j++)
      if (j < J) {
        uint32_t x0 = kv[j][0], x1 = kv[j][1], x2 = kv[j][2], x3 = kv[j][3];
        asm volatile("" : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));   // keeps the conversion (and its wait) out of the load's branch
        const int p = 4 * tid + 4 * NT * j;
        const uint32_t y[4] = {p + 0 < nr ? radix_key(__uint_as_float(x0)) : 0u,
                               p + 1 < nr ? radix_key(__uint_as_float(x1)) : 0u,
                               p + 2 < nr ? radix_key(__uint_as_float(x2)) : 0u,
                               p + 3 < nr ? radix_key(__uint_as_float(x3)) : 0u};
#pragma unroll
        for (int c = 0; c < 4; c++) {
          mn = min(mn, y[c] - 1u);
          mx = max(mx, y[c]);
        }
        reinterpret_cast<v4u*>(fk)[swz16(p >> 2)] = v4u{y[0], y[1], y[2], y[3]};
      }
    block_min_max(mn, mx, misc);                     // its barriers also publish fk
    STAMP(a, qrec, 1);
    int got = -1;
    done = select_all<ALL_MAX / NT, SHORT>(fk, nr, mn + 1u, mx, k, hist, misc, out, &got, stp);
    if (done && got != k && tid == 0) raise_error(ws, IDX_DERR_SELECT);
  } else if (!SHORT && path == PATH_CAND) {
    const int wact = (nr + C - 1) >> a.chunk_shift;
    const int upt = (wact + NT - 1) / NT;
    const uint64_t* erow = reinterpret_cast<const uint64_t*>(ws + a.off_ent) + (int64_t)grow * a.ent_stride * CAP_MAX;
    int m, cap, G;
    candidate_params(nr, C, k, &m, &cap, &G);
    const int SL = 32 * G;                           // slots a chunk
    __amdgpu_buffer_rsrc_t rent = make_rsrc(erow, (int64_t)wact * SL * 8);
    bool fast_rare = false;
    if (wact * SL <= NT * 16) {
      // One load of everything, piece-major: thread t holds the 16-byte slot pairs
      // u NT + t (u < 8) of the row's blocks, coalesced; pairs past the row's blocks read
      // zeros.  A chunk's block is 16 G pairs, so its header and maximum are pair u NT + t
      // of a thread with t % 16 G == 0 (lanes 0, 16, 32 or 48).  In the order (u, t, slot)
      // the candidates run in position order, so the selection works on the registers as
      // loaded: a header, maximum or empty slot has an upper word below every key, and the
      // keys below t* are dropped as absent.
      v4u sv[8];
#pragma unroll
      for (int u = 0; u < 8; u++)
        sv[u] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rent, (u * NT + tid) * 16, 0, 0));
      const int psh = G == 1 ? 4 : (G == 2 ? 5 : 6);  // pairs a block: 16 G = 1 << psh
      const bool hdr = (tid & ((1 << psh) - 1)) == 0;
      uint32_t t4[4] = {0u, 0u, 0u, 0u};
      if (hdr) {                                     // headers (zeros past the row: no effect)
#pragma unroll
        for (int u = 0; u < 8; u++) {
          const uint32_t tw = sv[u][0], flags = sv[u][1], cmax = sv[u][2];
          const bool ov = (flags >> 16) & 1u;
          t4[0] += ov ? 0u : (flags & 0xFFFFu);
          t4[1] = max(t4[1], ov ? 0u : tw);
          t4[2] = max(t4[2], cmax);
          t4[3] += ov ? 1u : 0u;
        }
      }
      header_reduce_sparse(t4, misc);
      STAMP(a, qrec, 1);
      if (t4[3] == 0u) {
        const uint32_t lo = t4[1] > 0x00800000u ? t4[1] : 0x00800000u;
        const uint32_t hi = t4[2] > lo ? t4[2] : lo;
        uint32_t kr[16], pr[16];
#pragma unroll
        for (int u = 0; u < 8; u++)
#pragma unroll
          for (int h2 = 0; h2 < 2; h2++) {
            const uint32_t key = sv[u][2 * h2 + 1];
            kr[2 * u + h2] = key >= lo ? key : 0u;
            pr[2 * u + h2] = sv[u][2 * h2];
          }
        uint32_t Tge;
        int rem;
        STAMPP(stp, 5);
        // the count of keys >= t* is unknown here: kth_select finds out whether k are present
        if (kth_select<16, true>(kr, 16, -1, lo, hi, k, hist, misc, &Tge, &rem, stp)) {
          STAMPP(stp, 3);
          const int got = emit_pieces<8, 2>(kr, pr, 8, Tge, rem, out, k, hist, stp);
          if (got != k && tid == 0) raise_error(ws, IDX_DERR_SELECT);
          done = true;
        }
      }
      if (!done) {
        // the rare cases from the registers as loaded: the chunk thresholds for a re-read
        // (bm, from the headers), the mass ties at the top (as in the general path below),
        // the hot-chunk set, else every published key into cand in position order (they
        // fit: at most 16 NT slots) and the re-read of the chunks that may hide keys
        __syncthreads();                             // misc may still be read
        // (without branches: a pair past the row's blocks read zeros, its entry of bm lies
        // past wact, where nothing reads, and a zero header never equals V, a key)
        if (hdr) {
#pragma unroll
          for (int u = 0; u < 8; u++) {
            const int w = (u * NT + tid) >> psh;
            bm[w] = ((sv[u][1] >> 16) & 1u) ? 0xFFFFFFFFu : sv[u][0];
            bm[6 * NT + w] = sv[u][1];
          }
        }
        if (t4[3] != 0u) {
          const uint32_t V = t4[2];
          uint32_t t2[4] = {0u, 0u, 0u, 0u};
          if (hdr) {
#pragma unroll
            for (int u = 0; u < 8; u++) t2[0] += sv[u][0] == V ? (sv[u][1] & 0xFFFFu) : 0u;
          }
          block_sum_max_max_sum(t2, misc);
          if ((int)t2[0] >= k) {
            emit_ordered(srow, nr, k, V + 1u, k, out, misc);
            done = true;
          }
        }
        if (!done && wact <= NT) {
          __syncthreads();                           // misc may still be read
          done = select_hot_chunks(ws, nr, k, wact, C, SL, erow, srow, cand, bm, hist, misc, out);
          if (!done) {
            // the blocks again (the candidate area and histograms were overwritten)
            __syncthreads();
            clear_hist(hist);
          }
        }
        if (!done) {
          // each thread's pairs made a run in position order first (slots [16 t, 16 t + 16))
          // through the candidate area at swz16 places; the scan below orders these reads
          // before the placement overwrites the area
          {
            v4u* const cq = reinterpret_cast<v4u*>(cand);
#pragma unroll
            for (int u = 0; u < 8; u++) cq[swz16(u * NT + tid)] = sv[u];
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 8; u++) sv[u] = cq[swz16(8 * tid + u)];
          }
          int c = 0;
#pragma unroll
          for (int u = 0; u < 8; u++)
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) c += sv[u][2 * h2 + 1] >= 0x00800000u ? 1 : 0;
          int tot;
          int o = block_excl_scan(c, misc, &tot);
#pragma unroll
          for (int u = 0; u < 8; u++)
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++)
              if (sv[u][2 * h2 + 1] >= 0x00800000u)
                cand[o++] = ((uint64_t)sv[u][2 * h2 + 1] << 32) | sv[u][2 * h2];
          done = rare_select(ws, nr, k, wact, tot, C, 0x00800000u, srow, cand, bm, hist, misc, out);
          fast_rare = true;                          // the general path would find the same
        }
      }
    }
    if (!done && !fast_rare) {
    // the chunk headers with their maxima (thread t: chunks t + NT u; past wact outside
    // the buffer resource), then the first gather batch, in flight together
    uint64_t e[2 * GQ];
    auto issue = [&](int b0) {
      if (G == 1) gather_issue<1>(rent, wact, b0, e);
      else if (G == 2) gather_issue<2>(rent, wact, b0, e);
      else gather_issue<4>(rent, wact, b0, e);
    };
    v4u hv[4];
#pragma unroll
    for (int u = 0; u < 4; u++)
      hv[u] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rent, (tid + NT * u) * SL * 8, 0, 0));
    issue(0);                                        // after the headers: their reduction overlaps it
    // the candidates published, t* = the largest t_w of the chunks that did not
    // overflow, the largest key of the row, the overflows; bm[w] keeps chunk w's t_w
    // (every key >= it is published) or ~0 for an overflowed chunk, for the rare path
    uint32_t t4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; u++) {
      if (u >= upt) break;
      const int w = tid + NT * u;
      if (w < wact) {
        const uint32_t tw = hv[u][0], flags = hv[u][1], cmax = hv[u][2];
        const bool ov = (flags >> 16) & 1u;
        t4[0] += ov ? 0u : (flags & 0xFFFFu);
        if (!ov) t4[1] = max(t4[1], tw);
        t4[2] = max(t4[2], cmax);
        t4[3] += ov ? 1u : 0u;
        bm[w] = ov ? 0xFFFFFFFFu : tw;
      }
    }
    block_sum_max_max_sum(t4, misc);
    STAMP(a, qrec, 1);
    // keys >= t* are all published (t* is at least every chunk's t_w): if k of them are
    // here, the k-th is among them and no chunk hides a key of the top k.  Only they are
    // gathered.  (0x00800000 is the smallest key of a finite score.)
    const uint32_t lo = t4[1] > 0x00800000u ? t4[1] : 0x00800000u;
    const uint32_t hi = t4[2] > lo ? t4[2] : lo;
    if (t4[3] != 0u) {
      // Mass ties at the top: V is the row's largest key.  A chunk whose threshold is V
      // counts exactly its keys equal to V (none is larger).  When such chunks hold k of
      // them in all, the list is the first k positions holding V, whatever the other
      // chunks hold (the ordered emission reads every position).
      const uint32_t V = t4[2];
      uint32_t t2[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 4; u++) {
        if (u >= upt) break;
        if (tid + NT * u < wact && hv[u][0] == V) t2[0] += hv[u][1] & 0xFFFFu;
      }
      block_sum_max_max_sum(t2, misc);
      if ((int)t2[0] >= k) {
        emit_ordered(srow, nr, k, V + 1u, k, out, misc);
        done = true;
      }
    }
    if (!done) {
      // the keys >= t* (not every published key: from about 1,024 chunks a row, the
      // published keys can pass the LDS capacity while those >= t* fit)
      int E = 0;
      bool fits = true;
      const int per_batch = batch_chunks(G);
      for (int b0 = 0; b0 < wact; b0 += per_batch) {
        if (b0 > 0) issue(b0);
        const int got = gather_place(e, lo, E, cand, misc);
        if (got < 0) {
          fits = false;
          break;
        }
        E += got;
      }
      STAMP(a, qrec, 2);
      if (fits) {
        pad_cand(cand, E);
        __syncthreads();
        if (t4[3] == 0u) {
          int got = -1;
          done = select_cand<FIN_ENT / NT>(cand, E, lo, hi, k, hist, misc, out, &got, stp);
          if (done && got != k && tid == 0) raise_error(ws, IDX_DERR_SELECT);
        }
        if (!done) {
          uint32_t glo = lo;
          bool ok = true;
          if (E < k) {
            // fewer than k keys >= t*: gather from a lower floor (chunk w then holds its keys
            // >= max(t_w, floor)).  Every published key when they fit (the highest T0 below,
            // so the fewest chunks to re-read); else the keys >= L, the (ceil(k / m) + 1)-th
            // largest t_w: the chunks at or above L publish at least m keys >= L each but for
            // the row's last (partial) chunk, so k in all.
            glo = 0x00800000u;
            if ((int)t4[0] > FIN_ENT) glo = header_floor(bm, wact, k, m, hist, misc, &ok);
            if (ok) {
              E = 0;
              for (int b0 = 0; b0 < wact && ok; b0 += per_batch) {
                if (wact > per_batch) issue(b0);       // else e still holds the one batch
                const int got = gather_place(e, glo, E, cand, misc);
                if (got < 0) ok = false;
                else E += got;
              }
            }
          }
          if (ok) done = rare_select(ws, nr, k, wact, E, C, glo, srow, cand, bm, hist, misc, out);
        }
      }
    }
    }
  }
  if (!done) {
    // ---- exact multi-pass select over the row's scores in memory
    __syncthreads();
    global_select_row(srow, nr, k, out, hist, misc);
  }
  STAMP(a, qrec, 4);
  return true;
}

// Launch 2.  OUT_SLOTS: each written list is then mapped to physical cache slots
// through the row's own page-table row: slot = page_table[row][p / 64] * 64 + p % 64,
// and -1 for -1 padding (or for a page id outside the pool, which the scoring launch has
// already reported).  OUT_TAGGED: the same slots, each stored as one 8-byte word
// tag << 32 | slot with a device-scope store, so that a consumer polling the word sees
// the old word or the whole new one.
// SHORT: every group's bound is at most ALL_MAX keys, so no row selects from candidate
// blocks; the kernel then carries only the paths such rows take, and its list stores
// mask off the unselected lanes (every slot of such a row holds a key).
constexpr int OUT_LIST = 0, OUT_SLOTS = 1, OUT_TAGGED = 2;
template <int OUT, bool SHORT>
__global__ __launch_bounds__(NT, 1) void select_kernel(const KArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  if (!select_row<SHORT>(a, smem) || OUT == OUT_LIST) return;
  __syncthreads();                                   // the list's stores, visible to the workgroup
  const uint32_t ge = a.grp[blockIdx.y];
  const int grow = (int)(ge & 0xFFFFFFu) + (int)blockIdx.x;
  const int32_t* lst = a.topk + (int64_t)grow * a.k;
  const int32_t* ptr = a.pt + (int64_t)grow * a.max_pages;
  for (int i = threadIdx.x; i < a.k; i += NT) {
    const int p = lst[i];
    int v = -1;
    if (p >= 0) {
      const int ph = ptr[p / PS];
      v = (ph >= 0 && ph < a.num_pages) ? ph * PS + (p % PS) : -1;
    }
    if constexpr (OUT == OUT_SLOTS) {
      a.slots[(int64_t)grow * a.k + i] = v;
    } else {
      const uint64_t word = ((uint64_t)a.tag << 32) | (uint32_t)v;
      __hip_atomic_store(a.tagged + (int64_t)grow * a.k + i, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Index-query preparation: one wave per (row, head), lane l holding dimensions 2 l and
// 2 l + 1 in f32.  RoPE reads each pair's partner through LDS, then the Hadamard
// transform runs as 7 butterfly stages (stride 1 within a lane, strides 2 .. 64 across
// lanes l and l ^ (stride / 2)), then a scale by 1/sqrt(128) and a round to bf16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);   // finite inputs
}

constexpr int PREP_WAVES = 4;   // waves (row, head pairs) a workgroup

__global__ __launch_bounds__(64 * PREP_WAVES) void prep_query_kernel(const uint32_t* qp, const float* cs, const float* sn,
                                                                     uint32_t* qo, int rows, int rope_dim,
                                                                     int interleaved) {
  __shared__ float buf[PREP_WAVES][D];
  const int lane = threadIdx.x & 63;
  const int wl = threadIdx.x >> 6;
  const int64_t task = (int64_t)blockIdx.x * PREP_WAVES + wl;        // row * H + head
  if (task >= (int64_t)rows * H) return;
  const int r = (int)(task / H);
  const uint32_t two = qp[task * (D / 2) + lane];                      // bf16 dims 2 l, 2 l + 1
  float v[2] = {__uint_as_float(two << 16), __uint_as_float(two & 0xFFFF0000u)};
  float* b = buf[wl];
  b[2 * lane] = v[0];
  b[2 * lane + 1] = v[1];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int half = rope_dim >> 1;
#pragma unroll
  for (int e = 0; e < 2; e++) {
    const int d = 2 * lane + e;
    if (d < rope_dim) {
      int i, partner;
      bool first;
      if (interleaved) {
        i = d >> 1;
        partner = d ^ 1;
        first = (d & 1) == 0;
      } else {
        first = d < half;
        i = first ? d : d - half;
        partner = first ? d + half : d - half;
      }
      const float c = cs[(int64_t)r * half + i], s = sn[(int64_t)r * half + i];
      const float x = b[d], y = b[partner];
      // the pair (a, b) becomes (a c - b s, a s + b c)
      v[e] = first ? fmaf(x, c, -(y * s)) : fmaf(y, s, x * c);
    }
  }
  float a0 = v[0] + v[1], a1 = v[0] - v[1];                            // stride 1
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {                                   // stride 2 m
    const float p0 = __shfl_xor(a0, m), p1 = __shfl_xor(a1, m);
    const bool hi = (lane & m) != 0;
    a0 = hi ? p0 - a0 : a0 + p0;
    a1 = hi ? p1 - a1 : a1 + p1;
  }
  constexpr float inv_sqrt_d = 0.08838834764831845f;                   // 1 / sqrt(128)
  qo[task * (D / 2) + lane] =
      (uint32_t)f32_to_bf16_rne(a0 * inv_sqrt_d) | ((uint32_t)f32_to_bf16_rne(a1 * inv_sqrt_d) << 16);
}

__global__ void fill_kernel(uint32_t* p, int64_t words, uint32_t magic) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < words) p[i] = (i == 0) ? magic : 0u;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
thread_local char g_hip_err[256] = "";
bool g_attr_done = false;

int hip_fail(hipError_t e) {
  snprintf(g_hip_err, sizeof g_hip_err, "%s", hipGetErrorString(e));
  return IDX_EHIP;
}

struct Plan {
  int pages_per_wg;   // P
  int chunk;          // keys per chunk
  int wg;             // chunks per group (grid x)
};

int pages_for(int max_keys) { return (max_keys + PS - 1) / PS; }

Plan plan_score(int max_keys) {
  const int pages = pages_for(max_keys);
  int need = (pages + 255) / 256;
  int P = 1;
  while (P < need && P < PMAX) P <<= 1;
  Plan pl;
  pl.pages_per_wg = P;
  pl.chunk = P * PS;
  pl.wg = pages > 0 ? (pages + P - 1) / P : 1;
  return pl;
}

Plan plan_topk(int max_keys) {
  Plan pl;
  pl.pages_per_wg = PMAX;
  pl.chunk = CMAX;
  pl.wg = max_keys > 0 ? (max_keys + CMAX - 1) / CMAX : 1;
  return pl;
}

struct WsLayout {
  uint64_t off_ent, off_stamps, total;
  int ent_stride;
};

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// The block area holds, per row, one block per chunk of any call of up to max_keys
// keys: plan_score gives at most min(256, pages) chunks while it uses fewer than 8 pages a
// chunk and ceil(pages / 8) beyond, plan_topk ceil(pages / 8); both bounds grow with
// max_keys, so a workspace sized for max_keys serves every smaller call.
WsLayout layout_for(int rows, int max_keys) {
  const int pages = pages_for(max_keys) > 0 ? pages_for(max_keys) : 1;
  const int lo = pages < 256 ? pages : 256, hi = (pages + PMAX - 1) / PMAX;
  const int stride = lo > hi ? lo : hi;
  WsLayout L;
  L.ent_stride = stride < 4 * NT ? stride : 4 * NT;     // rows with more chunks never publish
  L.off_ent = WS_HDR;
  L.off_stamps = align256(L.off_ent + (uint64_t)rows * L.ent_stride * CAP_MAX * 8);
  L.total = align256(L.off_stamps + STAMP_BYTES);
  return L;
}

int check_ptr(const void* p, uintptr_t align) {
  return (p != nullptr && (reinterpret_cast<uintptr_t>(p) % align) == 0) ? IDX_OK : IDX_EINVAL;
}

int validate_problem(const idx_problem* p) {
  if (!p) return IDX_EINVAL;
  if (p->heads != IDX_HEADS || p->dim != IDX_DIM || p->page_size != IDX_PAGE_SIZE) return IDX_EUNSUPPORTED;
  if (p->rows < 1 || p->num_req < 1 || !p->req_indptr) return IDX_EINVAL;
  if (p->num_req > IDX_MAX_REQ) return IDX_EUNSUPPORTED;
  if (p->rows > (1 << 24) - 1) return IDX_EUNSUPPORTED;
  if (p->req_indptr[0] != 0 || p->req_indptr[p->num_req] != p->rows) return IDX_EINVAL;
  int groups = 0;
  for (int j = 0; j < p->num_req; j++) {
    const int32_t r = p->req_indptr[j + 1] - p->req_indptr[j];
    if (r < 1) return IDX_EINVAL;
    groups += (r + IDX_GROUP_ROWS - 1) / IDX_GROUP_ROWS;
    if (groups > IDX_MAX_REQ) return IDX_EUNSUPPORTED;
  }
  if (p->num_pages < 1 || p->max_pages < 1 || p->max_keys < 0) return IDX_EINVAL;
  if (p->req_max_keys)
    for (int j = 0; j < p->num_req; j++)
      if (p->req_max_keys[j] < 0 || p->req_max_keys[j] > p->max_keys) return IDX_EINVAL;
  if ((int64_t)p->max_keys > (int64_t)p->max_pages * IDX_PAGE_SIZE) return IDX_EINVAL;
  if (p->max_keys > IDX_MAX_KEYS) return IDX_EUNSUPPORTED;
  if (check_ptr(p->q, 16) || check_ptr(p->w, 4) || check_ptr(p->k_cache, 16) || check_ptr(p->k_scale, 16) ||
      check_ptr(p->page_table, 4) || check_ptr(p->n_keys, 4))
    return IDX_EINVAL;
  return IDX_OK;
}

constexpr int SCORE_LDS = L_SCORE_END;
constexpr int SELECT_LDS = L_FIN_END;

int set_attrs() {
  if (g_attr_done) return IDX_OK;
  const void* fs[14] = {(const void*)score_kernel<1, false>,        (const void*)score_kernel<2, false>,
                        (const void*)score_kernel<4, false>,        (const void*)score_kernel<8, false>,
                        (const void*)score_kernel<1, true>,         (const void*)score_kernel<2, true>,
                        (const void*)score_kernel<4, true>,         (const void*)score_kernel<8, true>,
                        (const void*)select_kernel<OUT_LIST, false>, (const void*)select_kernel<OUT_SLOTS, false>,
                        (const void*)select_kernel<OUT_TAGGED, false>, (const void*)select_kernel<OUT_LIST, true>,
                        (const void*)select_kernel<OUT_SLOTS, true>, (const void*)select_kernel<OUT_TAGGED, true>};
  for (int i = 0; i < 14; i++) {
    const hipError_t e =
        hipFuncSetAttribute(fs[i], hipFuncAttributeMaxDynamicSharedMemorySize, i < 8 ? SCORE_LDS : SELECT_LDS);
    if (e != hipSuccess) return hip_fail(e);
  }
  g_attr_done = true;
  return IDX_OK;
}

// Launch 1 (grid: chunks x groups), then, when selecting, launch 2 (grid: rows of a
// group x groups) on the same stream.
int launch(const KArgs& args, int P, dim3 grid, bool score_launch, bool select_launch, hipStream_t st) {
  int rc = set_attrs();
  if (rc) return rc;
  if (score_launch) {
    const bool patch = args.nw_pos != nullptr;
    switch (P + (patch ? 16 : 0)) {
      case 1: hipLaunchKernelGGL((score_kernel<1, false>), grid, dim3(NT), SCORE_LDS, st, args); break;
      case 2: hipLaunchKernelGGL((score_kernel<2, false>), grid, dim3(NT), SCORE_LDS, st, args); break;
      case 4: hipLaunchKernelGGL((score_kernel<4, false>), grid, dim3(NT), SCORE_LDS, st, args); break;
      case 8: hipLaunchKernelGGL((score_kernel<8, false>), grid, dim3(NT), SCORE_LDS, st, args); break;
      case 17: hipLaunchKernelGGL((score_kernel<1, true>), grid, dim3(NT), SCORE_LDS, st, args); break;
      case 18: hipLaunchKernelGGL((score_kernel<2, true>), grid, dim3(NT), SCORE_LDS, st, args); break;
      case 20: hipLaunchKernelGGL((score_kernel<4, true>), grid, dim3(NT), SCORE_LDS, st, args); break;
      default: hipLaunchKernelGGL((score_kernel<8, true>), grid, dim3(NT), SCORE_LDS, st, args); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  if (select_launch) {
    const dim3 sg(IDX_GROUP_ROWS, grid.y);
    bool short_rows = true;
    for (unsigned g = 0; g < grid.y; g++) short_rows = short_rows && args.gmax[g] <= ALL_MAX;
    const int kind = (args.tagged ? OUT_TAGGED : (args.slots ? OUT_SLOTS : OUT_LIST)) + (short_rows ? 4 : 0);
    switch (kind) {
      case OUT_LIST: hipLaunchKernelGGL((select_kernel<OUT_LIST, false>), sg, dim3(NT), SELECT_LDS, st, args); break;
      case OUT_SLOTS: hipLaunchKernelGGL((select_kernel<OUT_SLOTS, false>), sg, dim3(NT), SELECT_LDS, st, args); break;
      case OUT_TAGGED: hipLaunchKernelGGL((select_kernel<OUT_TAGGED, false>), sg, dim3(NT), SELECT_LDS, st, args); break;
      case 4 + OUT_LIST: hipLaunchKernelGGL((select_kernel<OUT_LIST, true>), sg, dim3(NT), SELECT_LDS, st, args); break;
      case 4 + OUT_SLOTS: hipLaunchKernelGGL((select_kernel<OUT_SLOTS, true>), sg, dim3(NT), SELECT_LDS, st, args); break;
      default: hipLaunchKernelGGL((select_kernel<OUT_TAGGED, true>), sg, dim3(NT), SELECT_LDS, st, args); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  return IDX_OK;
}

void fill_common(KArgs& args, const WsLayout& L, void* ws) {
  args.ws = static_cast<uint8_t*>(ws);
  args.ent_stride = L.ent_stride;
  args.off_ent = L.off_ent;
  args.off_stamps = L.off_stamps;
}

int run_problem(const idx_problem* p, int32_t k, float* scores, int64_t ld, int32_t* topk, int32_t* slots,
                void* ws, size_t ws_bytes, void* stream, bool select, const idx_new_keys* nk = nullptr,
                bool scratch = false, uint64_t* tagged = nullptr, uint32_t tag = 0) {
  int rc = validate_problem(p);
  if (rc) return rc;
  if (!scores || ld < 1 || ld < (int64_t)p->max_keys) return IDX_EINVAL;
  if ((int64_t)p->rows > INT64_MAX / ld) return IDX_EINVAL;
  if (select) {
    if (k < 1 || k > IDX_KMAX || !topk) return IDX_EINVAL;
  } else {
    k = 1;
  }
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return IDX_EWORKSPACE;
  const WsLayout L = layout_for(p->rows, p->max_keys);
  if (ws_bytes < L.total) return IDX_EWORKSPACE;
  const Plan pl = plan_score(p->max_keys);
  KArgs args;
  memset(&args, 0, sizeof args);
  args.q = static_cast<const uint8_t*>(p->q);
  args.w = static_cast<const uint8_t*>(p->w);
  args.kc = p->k_cache;
  args.ks = p->k_scale;
  args.pt = p->page_table;
  args.nk = p->n_keys;
  args.scores = scores;
  args.topk = topk;
  args.slots = slots;
  args.tagged = tagged;
  args.tag = tag;
  args.ld = ld;
  args.rows = p->rows;
  args.max_pages = p->max_pages;
  args.max_keys = p->max_keys;
  args.num_pages = p->num_pages;
  args.k = k;
  args.chunk = pl.chunk;
  args.chunk_shift = 31 - __builtin_clz((unsigned)pl.chunk);
  args.mode = (select ? (MODE_SCORE | MODE_PUBLISH) : MODE_SCORE) | (scratch ? MODE_NOMAGIC : 0);
  fill_common(args, L, ws);
  if (nk) {
    args.nw_codes = nk->codes;
    args.nw_scales = nk->scales;
    args.nw_pos = nk->pos;
    args.kc_w = const_cast<uint8_t*>(p->k_cache);
    args.ks_w = const_cast<float*>(p->k_scale);
  }
  // a request of more than IDX_GROUP_ROWS rows is scored as consecutive groups of at
  // most IDX_GROUP_ROWS of its rows; each group walks the request's pages once
  int groups = 0;
  for (int j = 0; j < p->num_req; j++) {
    const int bound = p->req_max_keys ? p->req_max_keys[j] : p->max_keys;
    const int rows_j = p->req_indptr[j + 1] - p->req_indptr[j];
    for (int r0 = p->req_indptr[j]; r0 < p->req_indptr[j + 1]; r0 += IDX_GROUP_ROWS) {
      const int rn = p->req_indptr[j + 1] - r0 < IDX_GROUP_ROWS ? p->req_indptr[j + 1] - r0 : IDX_GROUP_ROWS;
      args.grp[groups] = (uint32_t)r0 | ((uint32_t)rn << 24);
      args.gmax[groups] = bound;
      args.req[groups] = (uint32_t)p->req_indptr[j] | ((uint32_t)rows_j << 24);
      groups++;
    }
  }
  return launch(args, pl.pages_per_wg, dim3(pl.wg, groups), true, select, static_cast<hipStream_t>(stream));
}

// Per-device address of `scratch`, looked up once per device with that device current.
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= MAX_DEVICES) return IDX_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255)) return IDX_EHIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return IDX_OK;
}

}  // namespace

extern "C" {

int idx_abi_version(void) { return IDX_ABI_VERSION; }

int idx_score_topk_noalloc(const idx_problem* p, int32_t k, float* scores, int64_t ld_scores, int32_t* topk,
                           void* stream) {
  // every host-side check of idx_score_topk first, then the size against the scratch
  int rc = validate_problem(p);
  if (rc) return rc;
  if (k < 1 || k > IDX_KMAX || !topk || !scores) return IDX_EINVAL;
  if (ld_scores < 1 || ld_scores < (int64_t)p->max_keys || (int64_t)p->rows > INT64_MAX / ld_scores) return IDX_EINVAL;
  if (layout_for(p->rows, p->max_keys).total > (uint64_t)IDX_NOALLOC_SCRATCH_BYTES) return IDX_ESCRATCH;
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc) return rc;
  return run_problem(p, k, scores, ld_scores, topk, nullptr, ws, IDX_NOALLOC_SCRATCH_BYTES, stream, true, nullptr,
                     true);
}

int idx_workspace_bytes(int32_t rows, int32_t max_keys, int32_t k, size_t* bytes) {
  if (!bytes || rows < 1 || rows > (1 << 24) - 1 || max_keys < 0 || k < 1 || k > IDX_KMAX) return IDX_EINVAL;
  if (max_keys > IDX_MAX_KEYS) return IDX_EUNSUPPORTED;
  *bytes = (size_t)layout_for(rows, max_keys).total;
  return IDX_OK;
}

int idx_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) || ws_bytes < WS_HDR || (ws_bytes & 255)) return IDX_EINVAL;
  const int64_t words = (int64_t)(ws_bytes / 4);
  const int blocks = (int)((words + 255) / 256);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(ws), words, WS_MAGIC);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? IDX_OK : hip_fail(e);
}

int idx_score(const idx_problem* p, float* scores, int64_t ld_scores, void* ws, size_t ws_bytes, void* stream) {
  return run_problem(p, 1, scores, ld_scores, nullptr, nullptr, ws, ws_bytes, stream, false);
}

int idx_score_topk(const idx_problem* p, int32_t k, float* scores, int64_t ld_scores, int32_t* topk, void* ws,
                   size_t ws_bytes, void* stream) {
  return run_problem(p, k, scores, ld_scores, topk, nullptr, ws, ws_bytes, stream, true);
}

int idx_score_topk_append(const idx_problem* p, const idx_new_keys* nk, int32_t k, float* scores,
                          int64_t ld_scores, int32_t* topk, void* ws, size_t ws_bytes, void* stream) {
  if (!nk || !nk->codes || !nk->scales || !nk->pos) return IDX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(nk->codes) & 15) || (reinterpret_cast<uintptr_t>(nk->scales) & 3) ||
      (reinterpret_cast<uintptr_t>(nk->pos) & 3))
    return IDX_EINVAL;
  const int rc = validate_problem(p);
  if (rc) return rc;
  for (int j = 0; j < p->num_req; j++)
    if (p->req_indptr[j + 1] - p->req_indptr[j] > NEW_MAX) return IDX_EUNSUPPORTED;
  return run_problem(p, k, scores, ld_scores, topk, nullptr, ws, ws_bytes, stream, true, nk);
}

int idx_score_topk_slots(const idx_problem* p, int32_t k, float* scores, int64_t ld_scores, int32_t* topk,
                         int32_t* slots, void* ws, size_t ws_bytes, void* stream) {
  if (!slots || (topk && slots == topk)) return IDX_EINVAL;
  return run_problem(p, k, scores, ld_scores, topk, slots, ws, ws_bytes, stream, true);
}

int idx_score_topk_tagged(const idx_problem* p, int32_t k, float* scores, int64_t ld_scores, int32_t* topk,
                          uint64_t* tagged, uint32_t tag, void* ws, size_t ws_bytes, void* stream) {
  if (!tagged || (reinterpret_cast<uintptr_t>(tagged) & 7)) return IDX_EINVAL;
  return run_problem(p, k, scores, ld_scores, topk, nullptr, ws, ws_bytes, stream, true, nullptr, false, tagged, tag);
}

int idx_topk(const float* scores, int64_t ld_scores, const int32_t* n_keys, int32_t rows, int32_t max_keys,
             int32_t k, int32_t* topk, void* ws, size_t ws_bytes, void* stream) {
  if (!scores || !n_keys || !topk || rows < 1 || rows > (1 << 24) - 1 || max_keys < 0) return IDX_EINVAL;
  if (max_keys > IDX_MAX_KEYS) return IDX_EUNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(scores) & 3) || (reinterpret_cast<uintptr_t>(n_keys) & 3)) return IDX_EINVAL;
  if (ld_scores < 1 || ld_scores < (int64_t)max_keys || (int64_t)rows > INT64_MAX / ld_scores) return IDX_EINVAL;
  if (k < 1 || k > IDX_KMAX) return IDX_EINVAL;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return IDX_EWORKSPACE;
  const WsLayout L = layout_for(rows, max_keys);
  if (ws_bytes < L.total) return IDX_EWORKSPACE;
  const Plan pl = plan_topk(max_keys);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // rows in groups of up to IDX_GROUP_ROWS, at most IDX_MAX_REQ groups per launch
  const int per_launch = IDX_MAX_REQ * IDX_GROUP_ROWS;
  for (int r0 = 0; r0 < rows; r0 += per_launch) {
    const int rn = (rows - r0) < per_launch ? (rows - r0) : per_launch;
    const int groups = (rn + IDX_GROUP_ROWS - 1) / IDX_GROUP_ROWS;
    KArgs args;
    memset(&args, 0, sizeof args);
    args.nk = n_keys;
    args.scores = const_cast<float*>(scores);
    args.topk = topk;
    args.ld = ld_scores;
    args.rows = rows;
    args.max_keys = max_keys;
    args.k = k;
    args.chunk = pl.chunk;
    args.chunk_shift = 31 - __builtin_clz((unsigned)pl.chunk);
    args.mode = MODE_PUBLISH;
    fill_common(args, L, ws);
    for (int gi = 0; gi < groups; gi++) {
      const int a0 = r0 + gi * IDX_GROUP_ROWS;
      const int an = (rows - a0) < IDX_GROUP_ROWS ? (rows - a0) : IDX_GROUP_ROWS;
      args.grp[gi] = (uint32_t)a0 | ((uint32_t)an << 24);
      args.gmax[gi] = max_keys;
    }
    // launch 1 only publishes candidates, which no row needs below ALL_MAX keys
    int rc = launch(args, pl.pages_per_wg, dim3(pl.wg, groups), max_keys > ALL_MAX, true, st);
    if (rc) return rc;
  }
  return IDX_OK;
}

int idx_prep_query(const void* q_pre, const float* cos_tab, const float* sin_tab, int32_t rows, int32_t rope_dim,
                   int32_t interleaved, void* q_out, void* stream) {
  if (!q_pre || !q_out || rows < 1 || rows > (1 << 24) - 1) return IDX_EINVAL;
  if (rope_dim < 0 || rope_dim > IDX_DIM || (rope_dim & 1) || (interleaved != 0 && interleaved != 1)) return IDX_EINVAL;
  if (rope_dim > 0 && (!cos_tab || !sin_tab)) return IDX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q_pre) & 3) || (reinterpret_cast<uintptr_t>(q_out) & 3) ||
      (reinterpret_cast<uintptr_t>(cos_tab) & 3) || (reinterpret_cast<uintptr_t>(sin_tab) & 3))
    return IDX_EINVAL;
  const int64_t tasks = (int64_t)rows * IDX_HEADS;
  const int blocks = (int)((tasks + PREP_WAVES - 1) / PREP_WAVES);
  hipLaunchKernelGGL(prep_query_kernel, dim3(blocks), dim3(64 * PREP_WAVES), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint32_t*>(q_pre), cos_tab, sin_tab, static_cast<uint32_t*>(q_out), rows,
                     rope_dim, interleaved);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? IDX_OK : hip_fail(e);
}

int idx_device_status(void* ws, size_t ws_bytes, void* stream, uint32_t* detail) {
  if (!ws || ws_bytes < WS_HDR) return IDX_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e);
  uint32_t hdr[2] = {0, 0};
  e = hipMemcpy(hdr, ws, sizeof hdr, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e);
  const uint32_t err = (hdr[0] != WS_MAGIC) ? (hdr[1] | IDX_DERR_WS) : hdr[1];
  if (detail) *detail = err;
  if (err) {
    uint32_t zero = 0;
    e = hipMemcpy(static_cast<uint8_t*>(ws) + WS_ERR_OFF, &zero, 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e);
    return IDX_EDEVICE;
  }
  return IDX_OK;
}

const char* idx_strerror(int code) {
  switch (code) {
    case IDX_OK: return "ok";
    case IDX_EINVAL: return "invalid argument";
    case IDX_EUNSUPPORTED: return "unsupported shape (heads, dim, page size, rows per request or request count)";
    case IDX_EWORKSPACE: return "workspace missing, misaligned or too small";
    case IDX_EHIP: return "HIP runtime error";
    case IDX_EDEVICE: return "device-side error recorded in the workspace";
    case IDX_ESCRATCH: return "problem too large for the static scratch of idx_score_topk_noalloc";
    default: return "unknown error code";
  }
}

const char* idx_last_hip_error(void) { return g_hip_err; }

#ifndef IDX_SOURCE_HASH
#define IDX_SOURCE_HASH "unknown"
#endif
// the marker string lets a build script read the hash from the file without loading it
static const char g_build_marker[] = "idx-source-sha256:" IDX_SOURCE_HASH;

const char* idx_build_hash(void) { return g_build_marker + 18; }

}  // extern "C"
