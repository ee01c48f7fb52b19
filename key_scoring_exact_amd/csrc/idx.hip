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
// one request.  It DMAs the group's bf16 queries and head weights into LDS, then the
// chunk's pages (16-byte global->LDS loads, three pages ahead of the compute, each
// key's 16-byte chunks XOR-swizzled so the operand reads below hit distinct banks).
// Each wave holds the A operands of one row (64 heads) in registers and runs bf16
// MFMA 32x32x16 over its tiles of 32 keys, the E4M3 codes widened to bf16 in
// registers (exact: every finite E4M3 value is a bf16 value).  FP8 MFMA is not
// used: on gfx950 it accumulates with an error near 1e-4 of the sum of |terms|,
// which would spend the whole score tolerance.  The tile loop is software
// pipelined: the MFMAs of one tile are issued, then the epilogue of the previous
// tile (ReLU, head weights, f32 head sum, key scale) and the widening of the next
// tile run on the VALU while the matrix core works.  For each row longer than
// ALL_MAX keys, the workgroup also publishes every key of its chunk at or above a
// local threshold t_w (the m-th largest of its 64 lane maxima), in position order,
// with a header word (t_w, count, overflow flag).
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

#include "idx.h"

namespace {

constexpr int H = IDX_HEADS;
constexpr int D = IDX_DIM;
constexpr int PS = IDX_PAGE_SIZE;
constexpr int GR = IDX_GROUP_ROWS;
constexpr int NT = 512;                 // threads per workgroup: 8 waves, two per SIMD
constexpr int NWAVE = NT / 64;
constexpr int PMAX = 8;                 // pages per workgroup at most
constexpr int CMAX = PMAX * PS;         // keys per chunk at most (512)
constexpr int LOOKAHEAD = 3;            // pages in flight ahead of the page being scored
constexpr int ALL_MAX = 24576;          // rows up to this many keys select from all scores at once
constexpr int FIN_ENT = 12288;          // candidate capacity of a finishing workgroup (the last 64
                                        // slots take the writes of empty lanes)
constexpr int BITMAP_KEYS = 131072;     // positions covered by the finisher's LDS bitmap
constexpr int CAP_MAX = 128;            // candidate slots per chunk and row
constexpr int LOAD_BATCH = 32;          // candidate loads in flight per thread
constexpr uint32_t WS_MAGIC = 0x1D5C0DE5u;

constexpr int MODE_SCORE = 1;           // compute scores (else read them from args.scores)
constexpr int MODE_PUBLISH = 2;         // publish each chunk's candidates for the selection launch

// LDS layout, scoring phase (bytes)
constexpr int L_KEYS = 0;                                   // [PMAX][64 keys][128 B], swizzled
constexpr int L_KSC = PMAX * PS * D;                        // [PMAX][64] f32 key scales
constexpr int L_SC = L_KSC + PMAX * PS * 4;                 // [GR][CMAX] f32 scores of the chunk
constexpr int L_Q = L_SC + GR * CMAX * 4;                   // [GR][64 heads][256 B] bf16 queries, swizzled
constexpr int L_W = L_Q + GR * H * D * 2;                   // [GR][64] bf16 head weights
constexpr int L_SCORE_END = L_W + GR * H * 2;
// LDS layout, finishing phase
constexpr int L_FK = 0;                                     // candidate keys: FIN_ENT
constexpr int L_FP = FIN_ENT * 4;                           // positions: FIN_ENT
constexpr int L_BM = FIN_ENT * 8;                           // bitmap: BITMAP_KEYS / 32 words
constexpr int HIST_WORDS = 4096 + 64;                       // one histogram: 4096 bins + 64 per-lane dummies
constexpr int L_HIST = L_BM + BITMAP_KEYS / 8;              // 2 histograms
constexpr int L_MISC = L_HIST + 2 * HIST_WORDS * 4;         // 64 u32 scratch
constexpr int L_CO = L_MISC + 64 * 4;                       // per chunk: candidate count (u8, 4 NT)
constexpr int L_GRP = L_CO + 4 * NT;                        // per group of 8 chunks: count, then base (2 x 256 u32)
constexpr int L_FIN_END = L_GRP + 2 * 256 * 4;
static_assert(BITMAP_KEYS / 8 >= 4 * NT * 8, "the failing-chunk list (2 words a chunk) fits the bitmap");
static_assert(ALL_MAX % NT == 0 && FIN_ENT % NT == 0, "register segments");
static_assert(CAP_MAX <= 128, "a chunk's candidates are gathered in at most two 64-slot groups");
static_assert(L_SCORE_END <= 160 * 1024 && L_FIN_END <= 160 * 1024, "LDS budget");

// workspace header (bytes)
constexpr int WS_MAGIC_OFF = 0;
constexpr int WS_ERR_OFF = 4;
constexpr int WS_HDR = 256;

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
  int32_t meta_stride;      // chunk slots per row (>= chunks of the longest row)
  int32_t ent_stride;       // chunk slots per row of the candidate area (min(meta_stride, 4 NT))
  uint64_t off_meta, off_ent;
  uint32_t grp[IDX_MAX_REQ];// row0 | nrows << 24
  int32_t gmax[IDX_MAX_REQ];// host bound on the keys of each group's rows
};

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, off) (reinterpret_cast<T*>(smem + (off)))

// ---------------------------------------------------------------------------
// memory helpers
// ---------------------------------------------------------------------------
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  int64_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0LL : (bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte global -> LDS DMA per lane: lane l writes LDS bytes [lds + 16 l, lds + 16 l + 16).
// Written as inline assembly so that the compiler neither tracks it nor inserts its own
// conservative waits before LDS reads; callers wait with explicit vmcnt counts.
__device__ inline void dma16(const void* gptr, uint32_t lds_wave_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_wave_base))
               : "memory");
}

__device__ inline void raise_error(uint8_t* ws, uint32_t bits) {
  __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(ws + WS_ERR_OFF), bits, __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
}

// Monotone map of a finite f32 score to an unsigned key (larger score, larger key);
// -0 is first folded into +0 so that equal reals get equal keys.  Finite scores map
// to keys >= 0x00800000, so 0 never denotes a real score.
__device__ inline uint32_t radix_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline int lane_id() { return (int)(threadIdx.x & 63); }
// the wave's index in the workgroup, as a wave-uniform (scalar) value
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// max(x, 0) of a float as one integer max of its bits: every negative float (and -0)
// is a negative int32, every positive float a positive one
__device__ inline float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// m-th largest of one value per lane (m >= 1): the largest t with #{v >= t} >= m.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t v, int m) {
  uint32_t t = 0;
  for (int b = 31; b >= 0; --b) {
    uint32_t cand = t | (1u << b);
    uint64_t bal = __ballot(v >= cand);
    if (__popcll(bal) >= m) t = cand;
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

// within each row of 16 lanes, lane 15 ends up holding the row's max / min / sum
__device__ __forceinline__ uint32_t row_max(uint32_t v) {
  v = max(v, dpp<0x111>(v, v));
  v = max(v, dpp<0x112>(v, v));
  v = max(v, dpp<0x114>(v, v));
  v = max(v, dpp<0x118>(v, v));
  return v;
}
__device__ __forceinline__ uint32_t row_min(uint32_t v) {
  v = min(v, dpp<0x111>(v, v));
  v = min(v, dpp<0x112>(v, v));
  v = min(v, dpp<0x114>(v, v));
  v = min(v, dpp<0x118>(v, v));
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

// Histogram increment of one key per lane (when `m`), aggregated over the wave for
// the bin of the first participating lane: radix digits of nearby scores pile into
// a few bins, and serialised LDS atomics on one address are the cost to avoid.
__device__ inline void hist_add(uint32_t* hist, bool m, uint32_t bin) {
  const uint64_t mb = __ballot(m);
  if (mb == 0) return;
  const int first = __ffsll((unsigned long long)mb) - 1;
  const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
  const bool same = m && bin == lb;
  const uint64_t sb = __ballot(same);
  if (lane_id() == first) atomicAdd(&hist[lb], (uint32_t)__popcll(sb));
  if (m && !same) atomicAdd(&hist[bin], 1u);
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
// holds kr[0 .. S) (slots past S hold 0); a zero key is absent.  Radix select over the
// bits below the common prefix of the smallest and largest key, in digits of up to 12
// bits from the top, histograms in LDS (hist: 2 x HIST_WORDS words).  Returns false
// if fewer than k keys are present.  Otherwise the top k (score descending, then
// position) are exactly: every key >= *Tge, and, when *rem > 0, also the first *rem
// keys equal to *T = *Tge - 1 in position order.  Absent keys never match a prefix
// once the first digit is fixed, and in the first pass they fall into bin 0, below
// every present key (a present key is >= 2^23 and the first digit starts at bit 21 or
// lower), so they are neither counted nor selected.  Slots are visited in groups of
// 8, skipping whole groups past S.  Every thread must call.
// ---------------------------------------------------------------------------
template <int SMAX>
__device__ __forceinline__ bool kth_regs(const uint32_t (&kr)[SMAX], int S, int k, uint32_t* hist, int* misc,
                                         uint32_t* Tge_out, int* rem_out) {
  static_assert(SMAX % 8 == 0, "slot groups of 8");
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  uint32_t mn = 0xFFFFFFFFu, mx = 0u, cnt = 0;
#pragma unroll
  for (int g = 0; g < SMAX / 8; g++) {
    if (g * 8 >= S) break;
#pragma unroll
    for (int jj = 0; jj < 8; jj++) {
      const uint32_t key = kr[g * 8 + jj];
      mn = min(mn, key - 1u);                         // absent keys wrap to 0xFFFFFFFF
      mx = max(mx, key);
      cnt += key != 0u ? 1u : 0u;
    }
  }
  mn = wave_min_u32(mn);                              // still key - 1 (absent: 0xFFFFFFFF)
  mx = wave_max_u32(mx);
  cnt = wave_sum_u32(cnt);
  uint32_t* red = reinterpret_cast<uint32_t*>(misc) + 16;
  if (lane == 0) {
    red[wv] = mn;
    red[NWAVE + wv] = mx;
    red[2 * NWAVE + wv] = cnt;
  }
  {
    const v4i z = {0, 0, 0, 0};
    v4i* h4 = reinterpret_cast<v4i*>(hist);
    h4[tid] = z;                                        // bins of the first buffer
    h4[tid + NT] = z;
  }
  __syncthreads();
  cnt = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; i++) {
    mn = min(mn, red[i]);
    mx = max(mx, red[NWAVE + i]);
    cnt += red[2 * NWAVE + i];
  }
  if ((int)cnt < k) return false;
  mn += 1u;                                           // the smallest present key
  if (mn == mx) {  // every key equal: the first k of them (all of them when cnt == k)
    *Tge_out = (int)cnt == k ? mn : mn + 1u;
    *rem_out = (int)cnt == k ? 0 : k;
    return true;
  }
  const int top = 31 - __clz(mn ^ mx);               // highest bit that differs
  uint32_t mask = (top == 31) ? 0u : ~((2u << top) - 1u);
  uint32_t prefix = mn & mask;
  const int nb = top + 1;                             // bits left to resolve
  const int npass = (nb + 11) / 12;
  const int wdef = (nb + npass - 1) / npass;
  int rem = k, shift = nb, buf = 0;
  const uint32_t dummy = 4096u + (uint32_t)lane;
  while (true) {
    const int width = wdef < shift ? wdef : shift;
    shift -= width;
    uint32_t* h = hist + buf * HIST_WORDS;
#pragma unroll
    for (int g = 0; g < SMAX / 8; g++) {
      if (g * 8 >= S) break;
#pragma unroll
      for (int jj = 0; jj < 8; jj++) {
        const uint32_t key = kr[g * 8 + jj];
        const uint32_t dg = __builtin_amdgcn_ubfe(key, (uint32_t)shift, (uint32_t)width);
        atomicAdd(&h[((key & mask) == prefix) ? dg : dummy], 1u);
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
    if (c == r && (shift == 0 || prefix != 0u)) {
      // every key of this digit is selected: the top k are exactly the keys >= prefix
      *Tge_out = prefix;
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
// the first rem such keys.  out[0 .. k) receives the selected positions pr[j] (stores
// of unselected slots go outside the buffer resource and are dropped).  Returns the
// number selected.  Every thread must call.
template <int SMAX>
__device__ __forceinline__ int emit_segments(const uint32_t (&kr)[SMAX], const uint32_t (&pr)[SMAX], int S,
                                             uint32_t Tge, int rem, int32_t* out, int k, int* misc) {
  constexpr int OOB = 0x7FFFFFF0;
  const uint32_t T = Tge - 1u;
  int gt = 0, eq = 0;
#pragma unroll
  for (int g = 0; g < SMAX / 8; g++) {
    if (g * 8 >= S) break;
#pragma unroll
    for (int jj = 0; jj < 8; jj++) gt += kr[g * 8 + jj] >= Tge ? 1 : 0;
  }
  if (rem > 0) {
#pragma unroll
    for (int g = 0; g < SMAX / 8; g++) {
      if (g * 8 >= S) break;
#pragma unroll
      for (int jj = 0; jj < 8; jj++) eq += kr[g * 8 + jj] == T ? 1 : 0;
    }
  }
  int tot;
  const int packed = block_excl_scan(gt | (eq << 16), misc, &tot);
  const int before_gt = packed & 0xFFFF, before_eq = packed >> 16;
  __amdgpu_buffer_rsrc_t ro = make_rsrc(out, (int64_t)k * 4);
  if (rem == 0) {
    int o4 = before_gt * 4;
#pragma unroll
    for (int g = 0; g < SMAX / 8; g++) {
      if (g * 8 >= S) break;
#pragma unroll
      for (int jj = 0; jj < 8; jj++) {
        const bool sel = kr[g * 8 + jj] >= Tge;
        __builtin_amdgcn_raw_buffer_store_b32(pr[g * 8 + jj], ro, sel ? o4 : OOB, 0, 0);
        o4 += sel ? 4 : 0;
      }
    }
  } else {
    int o = before_gt + (before_eq < rem ? before_eq : rem);
    int er = before_eq;
#pragma unroll
    for (int g = 0; g < SMAX / 8; g++) {
      if (g * 8 >= S) break;
#pragma unroll
      for (int jj = 0; jj < 8; jj++) {
        const uint32_t key = kr[g * 8 + jj];
        const bool e = key == T;
        const bool sel = key >= Tge || (e && er < rem);
        er += e ? 1 : 0;
        __builtin_amdgcn_raw_buffer_store_b32(pr[g * 8 + jj], ro, (sel && o < k) ? o * 4 : OOB, 0, 0);
        o += sel ? 1 : 0;
      }
    }
  }
  const int tg = tot & 0xFFFF, te = tot >> 16;
  return tg + (te < rem ? te : rem);
}

// Position of the rem-th set bit of bm[0 .. words) (1-based rem).  Every thread must call.
__device__ uint32_t nth_set_bit(const uint32_t* bm, int words, int rem, int* misc) {
  const int tid = threadIdx.x;
  const int wpt = (words + NT - 1) / NT;
  const int w0 = tid * wpt;
  int c = 0;
  for (int i = 0; i < wpt; i++) c += (w0 + i < words) ? __popc(bm[w0 + i]) : 0;
  int tot;
  const int before = block_excl_scan(c, misc, &tot);
  if (before < rem && rem <= before + c) {
    int need = rem - before;
    for (int i = 0; i < wpt; i++) {
      const uint32_t x = (w0 + i < words) ? bm[w0 + i] : 0u;
      const int pc = __popc(x);
      if (need <= pc) {
        uint32_t y = x;
        for (int s = 1; s < need; s++) y &= y - 1;
        misc[12] = (w0 + i) * 32 + (__ffs(y) - 1);
        break;
      }
      need -= pc;
    }
  }
  __syncthreads();
  const uint32_t r = (uint32_t)misc[12];
  __syncthreads();
  return r;
}

// Emit the set bits of bm[0 .. words) as ascending positions into out[0 .. kk).
// Returns how many bits were set.  Every thread must call.
__device__ int emit_bitmap(const uint32_t* bm, int words, int* misc, int32_t* out, int kk) {
  const int tid = threadIdx.x;
  const int wpt = (words + NT - 1) / NT;
  const int w0 = tid * wpt;
  int c = 0;
  for (int i = 0; i < wpt; i++) c += (w0 + i < words) ? __popc(bm[w0 + i]) : 0;
  int tot;
  int o = block_excl_scan(c, misc, &tot);
  for (int i = 0; i < wpt; i++) {
    if (w0 + i >= words) break;
    uint32_t x = bm[w0 + i];
    while (x) {
      const int b = __ffs(x) - 1;
      x &= x - 1;
      if (o < kk) out[o] = (w0 + i) * 32 + b;
      o++;
    }
  }
  return tot;
}

// Top k of the candidate set (K, P)[0 .. E) over positions [0, n), given the threshold
// (T, rem) of kth_regs, through a position bitmap (the candidates need not be in
// position order).  Returns the number emitted.  Every thread must call.
__device__ int select_explicit(const uint32_t* K, const uint32_t* P, int E, int n, int k, uint32_t T, int rem,
                               uint32_t* bm, int* misc, int32_t* out) {
  const int tid = threadIdx.x;
  const int words = (n + 31) >> 5;
  for (int i = tid; i < words; i += NT) bm[i] = 0;
  __syncthreads();
  int pos_cut = -1;                                   // keys equal to T at positions <= pos_cut
  if (rem > 0) {
    for (int e = tid; e < E; e += NT)
      if (K[e] == T) atomicOr(&bm[P[e] >> 5], 1u << (P[e] & 31));
    __syncthreads();
    pos_cut = (int)nth_set_bit(bm, words, rem, misc);
    for (int i = tid; i < words; i += NT) bm[i] = 0;
    __syncthreads();
  }
  for (int e = tid; e < E; e += NT) {
    const uint32_t key = K[e], p = P[e];
    if (key > T || (key == T && (int)p <= pos_cut)) atomicOr(&bm[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  return emit_bitmap(bm, words, misc, out, k);
}

// Exact top-k of row scores in global memory (n > k), one workgroup, LDS for the
// histogram only: radix select over all scores, then an ordered emission.
__device__ void global_select_row(const float* row, int n, int k, int32_t* out, uint32_t* hist, int* misc) {
  const int tid = threadIdx.x;
  __amdgpu_buffer_rsrc_t rs = make_rsrc(row, (int64_t)n * 4);
  uint32_t prefix = 0, mask = 0;
  int rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += NT * 8) {
      uint32_t v[8];
#pragma unroll
      for (int j = 0; j < 8; j++)
        v[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (base + j * NT + tid) * 4, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int p = base + j * NT + tid;
        const uint32_t key = radix_key(__uint_as_float(v[j]));
        hist_add(hist, p < n && (key & mask) == prefix, (key >> shift) & 255u);
      }
    }
    __syncthreads();
    find_digit(hist, 256, rem, misc);
    prefix |= (uint32_t)misc[8] << shift;
    mask |= 0xFFu << shift;
    rem = misc[9];
    __syncthreads();
  }
  const uint32_t T = prefix;
  int eq_carry = 0, sel_carry = 0;
  for (int base = 0; base < n; base += NT * 8) {
    const int p0 = base + tid * 8;
    uint32_t key[8];
#pragma unroll
    for (int j = 0; j < 8; j++)
      key[j] = radix_key(__uint_as_float(
          (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (p0 + j) * 4, 0, 0)));
    int ceq = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) ceq += (p0 + j < n && key[j] == T) ? 1 : 0;
    int eq_tot;
    int eq_before = block_excl_scan(ceq, misc, &eq_tot) + eq_carry;
    bool sel[8];
    int cs = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const bool valid = p0 + j < n;
      bool s = valid && key[j] > T;
      if (valid && key[j] == T) {
        s = eq_before < rem;
        eq_before++;
      }
      sel[j] = s;
      cs += s ? 1 : 0;
    }
    int sel_tot;
    int o = block_excl_scan(cs, misc, &sel_tot) + sel_carry;
#pragma unroll
    for (int j = 0; j < 8; j++)
      if (sel[j]) {
        if (o < k) out[o] = p0 + j;
        o++;
      }
    eq_carry += eq_tot;
    sel_carry += sel_tot;
  }
}

// m (lane-maximum rank used as the local threshold) and the candidate cap, from the
// row length n, chunk size C and k.  About k*C/n keys of a chunk reach the top k.
__device__ inline void candidate_params(int n, int C, int k, int* m, int* cap) {
  // k * C <= 2^20 and n >= 1: 32-bit arithmetic is exact
  const uint32_t lam = ((uint32_t)(k * C) + (uint32_t)n - 1u) / (uint32_t)n;
  int mm = (int)(lam + lam / 4u + 12u);
  mm = mm > 64 ? 64 : mm;
  int cc = 2 * mm + 16;
  cc = cc > C ? C : cc;
  cc = cc > CAP_MAX ? CAP_MAX : cc;
  *m = mm;
  *cap = cc;
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

// wait until this wave's DMAs of pages [0, x] are done, pages [0, issued) having
// been issued in page order, 2 DMA instructions per page per wave
__device__ inline void wait_pages_through(int x, int issued) {
  switch (2 * (issued - 1 - x)) {
    case 0: wait_vmcnt<0>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 10: wait_vmcnt<10>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// ---------------------------------------------------------------------------
// scoring of one chunk: scores of the group's rows land in sc_lds[row][0..C)
// TS = tile stride = waves per row (8 / R, 2 for R = 3); each wave scores one row.
// ---------------------------------------------------------------------------
template <int P, int TS>
__device__ __forceinline__ void score_chunk(const KArgs& a, uint8_t* smem, int R, int c, const int* phys) {
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  float* const sc_lds = LDS_PTR(float, L_SC);
  constexpr int T = (2 * P + TS - 1) / TS;      // tiles of 32 keys per wave
  const int lr = wv / TS;                       // this wave's row (>= R: an idle wave)
  const int toff = wv % TS;
  const bool live = lr < R;
  const int lrr = live ? lr : 0;
  const int g2 = lane >> 5;

  auto issue_page = [&](int j) {
    const uint8_t* pg = a.kc + (int64_t)phys[j] * (PS * D);
    const int kn = tid >> 3, cs = tid & 7;
    const int ch = cs ^ ((kn >> 1) & 7);
    dma16(pg + kn * D + ch * 16, lds0 + L_KEYS + j * (PS * D) + wv * 1024);
    // every wave issues the scale DMA (2 active lanes) so that all waves count alike
    if (lane < 2) dma16(a.ks + (int64_t)phys[j] * PS + wv * 8 + lane * 4, lds0 + L_KSC + j * (PS * 4) + wv * 32);
  };
  constexpr int L0 = (P < LOOKAHEAD) ? P : LOOKAHEAD;
#pragma unroll
  for (int j = 0; j < L0; j++) issue_page(j);
  // queries and head weights (issued first, waited for with the key counts) are in LDS
  __syncthreads();

  // A operands: bf16 MFMA 32x32x16, lane l supplies row l % 32 and 8 consecutive k of
  // its half l / 32.  K step s of half g covers d = 64 g + 8 s .. +8 (the keys use the
  // same mapping); M tile mt covers heads 32 mt .. +32.
  v8bf aq[2][8];
  float wr[2][16];
  {
    const uint8_t* qrow = smem + L_Q + lrr * (H * D * 2);
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

  // raw E4M3 words of this wave's tile i: key kn = (t & 1) * 32 + lane % 32, bytes
  // d = 64 g .. 64 g + 64 (4 swizzled 16-byte chunks)
  auto load_raw = [&](int i, uint32_t* kw) {
    const int t = toff + i * TS;
    const int j = t >> 1;
    const int kn = (t & 1) * 32 + (lane & 31);
    const uint8_t* kb = smem + L_KEYS + j * (PS * D) + kn * D;
    const int swz = (kn >> 1) & 7;
#pragma unroll
    for (int cc = 0; cc < 4; cc++) {
      const v4i x = *reinterpret_cast<const v4i*>(kb + (((4 * g2 + cc) ^ swz) << 4));
      kw[4 * cc + 0] = (uint32_t)x[0];
      kw[4 * cc + 1] = (uint32_t)x[1];
      kw[4 * cc + 2] = (uint32_t)x[2];
      kw[4 * cc + 3] = (uint32_t)x[3];
    }
  };
  // 8 E4M3 codes of K step st, widened exactly to bf16
  auto widen = [&](const uint32_t* kw, int st) -> v8bf {
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[2 * st], 1.0f, false);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[2 * st], 1.0f, true);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[2 * st + 1], 1.0f, false);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[2 * st + 1], 1.0f, true);
    return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  };
  auto epilogue = [&](int i, const v16f& acc0, const v16f& acc1) {
    const int t = toff + i * TS;
    const int j = t >> 1;
    const int kn = (t & 1) * 32 + (lane & 31);
    const float ksv = ksl[j * PS + kn];
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      s0 = fmaf(wr[0][q], relu(acc0[q]), s0);
      s1 = fmaf(wr[1][q], relu(acc1[q]), s1);
    }
    float sum = s0 + s1;
    sum += __shfl_xor(sum, 32);
    if (live && lane < 32) sc_lds[lr * CMAX + t * 32 + lane] = sum * ksv + 0.0f;
  };
  // the highest page any wave reads at iteration i
  auto page_of_iter = [&](int i) { return ((i * TS + TS - 1) >> 1) < P - 1 ? ((i * TS + TS - 1) >> 1) : P - 1; };

  int issued = L0;
  auto ensure_page = [&](int x) {
    // pages [0, x] issued and landed (all waves' parts), then LOOKAHEAD more in flight
#pragma unroll
    for (int j = 0; j < P; j++)
      if (j >= issued && j <= x) issue_page(j);
    if (issued < x + 1) issued = x + 1;
    wait_pages_through(x, issued);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < P; j++)
      if (j >= issued && j <= x + LOOKAHEAD) issue_page(j);
    if (issued < x + LOOKAHEAD + 1) issued = (x + LOOKAHEAD + 1 < P) ? x + LOOKAHEAD + 1 : P;
  };

  ensure_page(page_of_iter(0));
  uint32_t kw_cur[16], kw_nxt[16];
  load_raw(0, kw_cur);
  v16f accp0 = {}, accp1 = {};
#pragma unroll
  for (int i = 0; i < T; i++) {
    if (i + 1 < T) ensure_page(page_of_iter(i + 1));
    // one scheduling region: this tile's MFMAs, the previous tile's epilogue and the
    // next tile's raw loads, interleaved so the VALU runs while the matrix core works
    if (i + 1 < T) load_raw(i + 1, kw_nxt);
    v16f acc0 = {}, acc1 = {};
#pragma unroll
    for (int st = 0; st < 8; st++) {
      const v8bf b = widen(kw_cur, st);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[0][st], b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[1][st], b, acc1, 0, 0, 0);
    }
    if (i > 0) epilogue(i - 1, accp0, accp1);
#pragma unroll
    for (int q = 0; q < 4; q++) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS reads first
#pragma unroll
    for (int q = 0; q < 16; q++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                             // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);                             // 6 VALU
    }
    accp0 = acc0;
    accp1 = acc1;
#pragma unroll
    for (int q = 0; q < 16; q++) kw_cur[q] = kw_nxt[q];
  }
  epilogue(T - 1, accp0, accp1);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
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

// t[0] and t[2] summed, t[1] maxed over the workgroup.  Every thread must call.
__device__ __forceinline__ void block_sum_max_sum(uint32_t (&t)[3], int* misc) {
  const uint32_t a = wave_sum_u32(t[0]), b = wave_max_u32(t[1]), c = wave_sum_u32(t[2]);
  const int wv = wave_id();
  if (lane_id() == 0) {
    misc[wv] = (int)a;
    misc[NWAVE + wv] = (int)b;
    misc[2 * NWAVE + wv] = (int)c;
  }
  __syncthreads();
  uint32_t sa = 0, mb = 0, sc = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; i++) {
    sa += (uint32_t)misc[i];
    mb = max(mb, (uint32_t)misc[NWAVE + i]);
    sc += (uint32_t)misc[2 * NWAVE + i];
  }
  __syncthreads();
  t[0] = sa;
  t[1] = mb;
  t[2] = sc;
}

// The row's published candidates into LDS in position order: FK[e] = key, FP[e] =
// position for e < E.  Chunk w's candidates sit at erow[w * CAP_MAX + s] for s < its
// count cnt8[w] <= 64 SLOTS.  Chunks come in groups of 8: group g starts at position-
// ordered offset gbase[g], so candidate s of chunk w goes to slot gbase[w / 8] + (counts
// of the chunks before w in its group) + s, known before anything is loaded.  In batch
// b wave v takes the GPB groups b NWAVE GPB + v GPB + j (j < GPB), issuing one 64-slot
// load per lane and chunk for all of them before the first use; slots past a count
// point outside the buffer resource (no traffic, zero result) and write into the last
// 64 LDS slots, which E <= FIN_ENT - 64 leaves free.  No barrier inside.
template <int SLOTS>
__device__ __forceinline__ void gather_candidates(const uint64_t* erow, int wact, const uint8_t* cnt8,
                                                  const uint32_t* gbase, uint32_t* FK, uint32_t* FP) {
  constexpr int OOB = 0x7FFFFFF0;
  constexpr int GPB = 4 / SLOTS;                        // groups a wave and batch
  constexpr int L = GPB * 8 * SLOTS;                    // loads a lane and batch (32)
  const int lane = lane_id(), wv = wave_id();
  __amdgpu_buffer_rsrc_t rent = make_rsrc(erow, (int64_t)wact * CAP_MAX * 8);
  const int groups = (wact + 7) / 8;
  const int dummy = FIN_ENT - 64 + lane;
#pragma unroll 1
  for (int gb = wv * GPB; gb < groups; gb += NWAVE * GPB) {
    int off[L], at[L];
#pragma unroll
    for (int j = 0; j < GPB; j++) {
      const int g = gb + j;
      const int w0 = g * 8;
      // group g's 8 chunk counts (one byte a chunk; bytes past wact are 0) and its base,
      // as wave-uniform values
      const bool live = g < groups;
      const v2i_t cq = live ? *reinterpret_cast<const v2i_t*>(cnt8 + w0) : v2i_t{0, 0};
      const uint32_t c0 = (uint32_t)__builtin_amdgcn_readfirstlane(cq[0]);
      const uint32_t c1 = (uint32_t)__builtin_amdgcn_readfirstlane(cq[1]);
      int base = live ? __builtin_amdgcn_readfirstlane((int)gbase[g]) : 0;
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const int cu = (int)(((q < 4 ? c0 : c1) >> ((q & 3) * 8)) & 0xFFu);
#pragma unroll
        for (int s2 = 0; s2 < SLOTS; s2++) {
          const int sl = s2 * 64 + lane;
          const bool v = sl < cu;
          off[(j * 8 + q) * SLOTS + s2] = v ? ((w0 + q) * CAP_MAX + sl) * 8 : OOB;
          at[(j * 8 + q) * SLOTS + s2] = v ? base + sl : dummy;
        }
        base += cu;
      }
    }
    uint64_t e[L];
#pragma unroll
    for (int i = 0; i < L; i++)
      e[i] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rent, off[i], 0, 0));
#pragma unroll
    for (int i = 0; i < L; i++) {
      FK[at[i]] = (uint32_t)(e[i] >> 32);
      FP[at[i]] = (uint32_t)e[i];
    }
  }
}

// Top k of the E candidates FK[0 .. E) (with positions FP[e], or e itself when
// IMPLICIT), laid out in position order; candidates below lo do not count.  Thread t
// holds candidates [t S, t S + S), S odd so that the strided LDS reads are free of
// bank conflicts.  Returns false (writing nothing) when fewer than k candidates count.
// Every thread must call.
template <int SMAX, bool IMPLICIT>
__device__ __forceinline__ bool select_emit(const uint32_t* FK, const uint32_t* FP, int E, uint32_t lo, int k,
                                            uint32_t* hist, int* misc, int32_t* out, int* got) {
  const int S = ((E + NT - 1) / NT) | 1;
  const int e0 = threadIdx.x * S;
  uint32_t kr[SMAX], pr[SMAX];
#pragma unroll
  for (int j = 0; j < SMAX; j++) {
    kr[j] = 0u;
    pr[j] = 0u;
  }
#pragma unroll
  for (int g = 0; g < SMAX / 8; g++) {
    if (g * 8 >= S) break;
#pragma unroll
    for (int jj = 0; jj < 8; jj++) {
      const int j = g * 8 + jj, e = e0 + j;
      const bool v = j < S && e < E;
      const uint32_t key = v ? FK[e] : 0u;
      kr[j] = key >= lo ? key : 0u;
      pr[j] = IMPLICIT ? (uint32_t)e : (v ? FP[e] : 0u);
    }
  }
  uint32_t Tge;
  int rem;
  if (!kth_regs<SMAX>(kr, S, k, hist, misc, &Tge, &rem)) return false;
  *got = emit_segments<SMAX>(kr, pr, S, Tge, rem, out, k, misc);
  return true;
}

// Candidate path when the certificate fails.  T0 = the k-th candidate (if there are
// k); every chunk whose local threshold t_w (tw[w], 0xFFFFFFFF when it published
// nothing) is above T0 is re-read from the row's scores for its unpublished keys >= T0,
// after which every key >= T0 of the row is a candidate, and the top k is taken from
// that set through a position bitmap.  Returns true when it selected, false to fall
// back to the multi-pass select over memory.  Every thread must call.
__device__ __forceinline__ bool rare_select(uint8_t* ws, int nr, int k, int wact, int E, int C,
                                            __amdgpu_buffer_rsrc_t rs, uint32_t* FK, uint32_t* FP, uint32_t* bm,
                                            uint32_t* hist, int* misc, int32_t* out) {
  const int tid = threadIdx.x;
  constexpr int SR = 32;
  uint32_t kr[SR];
  auto load_keys = [&](int n_ent) {
    int S = (n_ent + NT - 1) / NT;
    S |= 1;
    const int e0 = tid * S;
#pragma unroll
    for (int j = 0; j < SR; j++) kr[j] = (j < S && e0 + j < n_ent) ? FK[e0 + j] : 0u;
    return S;
  };
  uint32_t T = 0;
  int rem = 0;
  const int S0 = load_keys(E);
  const bool full = E >= k && kth_regs<SR>(kr, S0, k, hist, misc, &T, &rem);
  // the k-th largest candidate is Tge - 1 when ties are cut, else at least Tge
  const uint32_t lowT = full ? (rem > 0 ? T - 1u : T) : 0u;
  // failing chunks listed in bm[4 NT ...] (tw[] occupies bm[0 .. 4 NT))
  uint32_t* fl = bm + 4 * NT;
  int nfail = 0;
  for (int w0 = 0; w0 < wact; w0 += NT) {
    const int w = w0 + tid;
    const bool f = w < wact && (!full || bm[w] > lowT);
    int tot;
    const int o = block_excl_scan(f ? 1 : 0, misc, &tot);
    if (f) fl[nfail + o] = (uint32_t)w;
    nfail += tot;
  }
  __syncthreads();
  int Ecur = E;
#pragma unroll 1
  for (int f = 0; f < nfail; f++) {
    const uint32_t w = fl[f];
    const uint32_t twf = bm[w];
    const int p0 = (int)w * C;
#pragma unroll 1
    for (int base = 0; base < C; base += NT) {
      const int p = p0 + base + tid;
      bool take = false;
      uint32_t key = 0;
      if (base + tid < C && p < nr) {
        key = radix_key(__uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, p * 4, 0, 0)));
        take = key >= lowT && key < twf;
      }
      int tot;
      const int oo = block_excl_scan(take ? 1 : 0, misc, &tot);
      if (Ecur + tot > FIN_ENT) return false;
      if (take) { FK[Ecur + oo] = key; FP[Ecur + oo] = (uint32_t)p; }
      Ecur += tot;
    }
  }
  __syncthreads();
  if (Ecur < k) return false;
  const int S1 = load_keys(Ecur);
  if (!kth_regs<SR>(kr, S1, k, hist, misc, &T, &rem)) return false;
  // select_explicit takes keys > T - 1 (>= Tge) and the first rem keys equal to Tge - 1
  const int got = select_explicit(FK, FP, Ecur, nr, k, T - 1u, rem, bm, misc, out);
  if (got != k && tid == 0) raise_error(ws, IDX_DERR_SELECT);
  return true;
}

// x[u] for a runtime u < 4 without indexing registers
__device__ inline int pick4(const int (&x)[4], int u) {
  return u == 0 ? x[0] : u == 1 ? x[1] : u == 2 ? x[2] : x[3];
}

// Exclusive scan of v and maximum of m over the workgroup.  Every thread must call.
__device__ inline int block_scan_max(int v, uint32_t m, int* misc, int* total, uint32_t* mall) {
  const int lane = lane_id(), wv = wave_id();
  const int x = wave_incl_scan(v);
  m = wave_max_u32(m);
  if (lane == 63) misc[wv] = x;
  if (lane == 0) misc[NWAVE + wv] = (int)m;
  __syncthreads();
  int before = 0, tot = 0;
  uint32_t mx = 0;
  const v4i* m4 = reinterpret_cast<const v4i*>(misc);
  const v4i s0 = m4[0], s1 = m4[1], x0 = m4[2], x1 = m4[3];
  const int sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  const int xv[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
  for (int i = 0; i < NWAVE; i++) {
    before += (i < wv) ? sv[i] : 0;
    tot += sv[i];
    mx = mx > (uint32_t)xv[i] ? mx : (uint32_t)xv[i];
  }
  __syncthreads();
  *total = tot;
  *mall = mx;
  return x - v + before;
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
template <int P>
__global__ __launch_bounds__(NT, 1) void score_kernel(const KArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const int c = blockIdx.x;
  const int g = blockIdx.y;
  const uint32_t ge = a.grp[g];
  const int row0 = (int)(ge & 0xFFFFFFu);
  const int R = (int)(ge >> 24);
  const int C = a.chunk;
  const int chunk_base = c * C;
  uint8_t* const ws = a.ws;

  const int gbound = a.gmax[g];
  if (c > 0 && chunk_base >= gbound) return;      // beyond every row of this group
  const bool do_score = (a.mode & MODE_SCORE) != 0;
  const bool do_pub = (a.mode & MODE_PUBLISH) != 0;
  if (*reinterpret_cast<const uint32_t*>(ws + WS_MAGIC_OFF) != WS_MAGIC) {
    if (tid == 0 && c == 0 && g == 0) raise_error(ws, IDX_DERR_WS);
    return;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  if (do_score) {
    // Queries and head weights of the group's rows into LDS first (2R + 1 DMA per
    // wave); their latency overlaps the n_keys / page-table load below.  Head h's 16
    // chunks of 16 bytes sit at chunk positions c ^ (h & 15), so the A-operand reads
    // (16 lanes on 16 heads, same chunk) hit distinct banks.
    for (int ii = wv * 2 * R; ii < (wv + 1) * 2 * R; ii++) {
      const int rr = ii >> 4;
      const int s16 = (ii & 15) * 64 + lane;
      const int h = s16 >> 4, cpos = s16 & 15;
      const int ch = cpos ^ (h & 15);
      dma16(a.q + ((int64_t)(row0 + rr) * H * D + h * D) * 2 + ch * 16, lds0 + L_Q + rr * (H * D * 2) + (ii & 15) * 1024);
    }
    if (lane < 8) dma16(a.w + (int64_t)(row0 + (wv % R)) * H * 2 + lane * 16, lds0 + L_W + (wv % R) * (H * 2));
  }
  // n_keys of the group's rows and the chunk's page ids of every row, in one load
  // (lanes [0, R): n_keys; lanes [8, 8 + R*P): page_table[row][c*P + j])
  int ld_lane = 0;
  if (lane < R) {
    ld_lane = a.nk[row0 + lane];
  } else if (do_score && lane >= 8 && lane < 8 + R * P) {
    const int i = (lane - 8) / P, j = (lane - 8) % P;
    if (c * P + j < a.max_pages) ld_lane = a.pt[(int64_t)(row0 + i) * a.max_pages + c * P + j];
  }
  wait_vmcnt<0>();

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
  uint64_t* const meta = reinterpret_cast<uint64_t*>(ws + a.off_meta);
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
    if (R == 1) score_chunk<P, 8>(a, smem, R, c, phys);
    else if (R == 2) score_chunk<P, 4>(a, smem, R, c, phys);
    else score_chunk<P, 2>(a, smem, R, c, phys);
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

  // ---------------- publish (wave i handles row i) -----------------------------------
  if (do_pub && wv < R) {
    const int i = wv;
    const int nr = n[i];
    const int nv = nr - chunk_base;
    if (nv > 0 && row_path(nr, k, shift) == PATH_CAND) {
      // candidates: every key of the chunk >= t_w (the m-th largest of the 64 lane
      // maxima), as (key << 32 | position), in ascending position order; a chunk with
      // more than cap of them publishes none and is flagged
      const int grow = row0 + i;
      int m, cap;
      candidate_params(nr, C, k, &m, &cap);
      uint32_t key[8];
      uint32_t lmax = 0;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int p = lane * 8 + j;
        key[j] = (p < nv && p < C) ? radix_key(sc_lds[i * CMAX + p]) : 0u;
        lmax = lmax > key[j] ? lmax : key[j];
      }
      const uint32_t thr = wave_kth_largest(lmax, m);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < 8; j++) cnt += (key[j] != 0u && key[j] >= thr) ? 1 : 0;
      const int incl = wave_incl_scan(cnt);
      const int total = __shfl(incl, 63);
      uint32_t cw;
      if (total > cap) {
        cw = 1u << 16;
      } else {
        int o = incl - cnt;
        uint64_t* dst = ent + ((int64_t)grow * a.ent_stride + c) * CAP_MAX;
#pragma unroll
        for (int j = 0; j < 8; j++)
          if (key[j] != 0u && key[j] >= thr) {
            dst[o] = ((uint64_t)key[j] << 32) | (uint32_t)(chunk_base + lane * 8 + j);
            o++;
          }
        cw = (uint32_t)total;
      }
      if (lane == 0) meta[(int64_t)grow * a.meta_stride + c] = ((uint64_t)thr << 32) | cw;
    }
  }

  // ---------------- scores out -------------------------------------------------------
  if (do_score) {
#pragma unroll
    for (int i = 0; i < GR; i++) {
      if (i >= R) break;
      const int nv = n[i] - chunk_base;
      float* dst = a.scores + (int64_t)(row0 + i) * a.ld + chunk_base;
      __amdgpu_buffer_rsrc_t rs = make_rsrc(dst, (int64_t)(nv > 0 ? (nv < C ? nv : C) : 0) * 4);
      for (int p = tid; p < C; p += NT)
        if (p < nv) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc_lds[i * CMAX + p]), rs, p * 4, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Launch 2: workgroup (i, g) selects row i of request g.  Launch 1 has ended, so its
// scores and candidates are in memory.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT, 1) void select_kernel(const KArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = wave_id();
  const uint32_t ge = a.grp[blockIdx.y];
  const int R = (int)(ge >> 24);
  const int i = blockIdx.x;
  if (i >= R) return;
  const int grow = (int)(ge & 0xFFFFFFu) + i;
  uint8_t* const ws = a.ws;
  if (*reinterpret_cast<const uint32_t*>(ws + WS_MAGIC_OFF) != WS_MAGIC) {
    if (tid == 0 && i == 0 && blockIdx.y == 0) raise_error(ws, IDX_DERR_WS);
    return;
  }
  const int gbound = a.gmax[blockIdx.y];
  int nr = __builtin_amdgcn_readfirstlane(a.nk[grow]);
  if (nr < 0 || nr > gbound) {
    if (tid == 0) raise_error(ws, IDX_DERR_NKEYS);
    nr = nr < 0 ? 0 : gbound;
  }
  const int k = a.k, C = a.chunk;
  int32_t* out = a.topk + (int64_t)grow * k;
  const int path = row_path(nr, k, a.chunk_shift);
  if (path == PATH_NONE) {
    for (int p = tid; p < k; p += NT) out[p] = p < nr ? p : -1;
    return;
  }
  int* misc = LDS_PTR(int, L_MISC);
  uint32_t* hist = LDS_PTR(uint32_t, L_HIST);
  uint32_t* FK = LDS_PTR(uint32_t, L_FK);
  uint32_t* FP = LDS_PTR(uint32_t, L_FP);
  uint32_t* bm = LDS_PTR(uint32_t, L_BM);
  const float* srow = a.scores + (int64_t)grow * a.ld;
  __amdgpu_buffer_rsrc_t rs = make_rsrc(srow, (int64_t)nr * 4);
  bool done = false;
  if (path == PATH_ALL) {
    // every key of the row into LDS (FK[p] for position p), coalesced: thread t reads
    // positions t + NT j
    constexpr int JA = ALL_MAX / NT;
    const int J = (nr + NT - 1) / NT;
    uint32_t kv[JA];
#pragma unroll
    for (int j = 0; j < JA; j++)
      kv[j] = j < J ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, tid * 4, j * NT * 4, 0) : 0u;
#pragma unroll
    for (int j = 0; j < JA; j++)
      if (j < J) FK[j * NT + tid] = radix_key(__uint_as_float(kv[j]));
    __syncthreads();
    int got = -1;
    done = select_emit<56, true>(FK, FP, nr, 0u, k, hist, misc, out, &got);
    if (done && got != k && tid == 0) raise_error(ws, IDX_DERR_SELECT);
  } else if (path == PATH_CAND) {
    // ---- chunk words: thread t reads the words of chunks t + NT u (u < upt)
    const int wact = (nr + C - 1) >> a.chunk_shift;
    const int upt = (wact + NT - 1) / NT;
    const uint64_t* mrow = reinterpret_cast<const uint64_t*>(ws + a.off_meta) + (int64_t)grow * a.meta_stride;
    const uint64_t* erow = reinterpret_cast<const uint64_t*>(ws + a.off_ent) + (int64_t)grow * a.ent_stride * CAP_MAX;
    __amdgpu_buffer_rsrc_t rmeta = make_rsrc(mrow, (int64_t)wact * 8);
    uint64_t mv[4];
#pragma unroll
    for (int u = 0; u < 4; u++)
      mv[u] = (u < upt) ? __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rmeta, (tid + NT * u) * 8, 0, 0))
                        : 0ull;
    int m_unused, cap;
    candidate_params(nr, C, k, &m_unused, &cap);
    uint8_t* cnt8 = LDS_PTR(uint8_t, L_CO);
    uint32_t* gcnt = LDS_PTR(uint32_t, L_GRP);
    uint32_t* gbase = gcnt + 256;
    if (tid < 256) gcnt[tid] = 0;
    __syncthreads();
    // per chunk: its count (cnt8), per group of 8 chunks: the count (gcnt); bm[w] =
    // t_w (0xFFFFFFFF: overflowed, published nothing) for the rare path; E = the
    // candidates published, t* = the largest t_w, whether any chunk overflowed
    uint32_t pub = 0, tmax = 0, ovs = 0;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int w = tid + NT * u;
      if (u >= upt) break;
      const uint32_t lw = (uint32_t)mv[u];
      const bool live = w < wact;
      const bool ov = live && ((lw >> 16) & 1u);
      const uint32_t cu = (live && !ov) ? (lw & 0xFFFFu) : 0u;
      const uint32_t twu = (uint32_t)(mv[u] >> 32);
      cnt8[w] = (uint8_t)cu;                       // w < 4 NT: bytes past wact read as 0
      if (cu) atomicAdd(&gcnt[w >> 3], cu);
      pub += cu;
      ovs += ov ? 1u : 0u;
      if (live && !ov) tmax = max(tmax, twu);
      if (live) bm[w] = ov ? 0xFFFFFFFFu : twu;
    }
    uint32_t t3[3] = {pub, tmax, ovs};
    block_sum_max_sum(t3, misc);
    const int E = (int)t3[0];
    // keys >= t* are all published (t* is at least every chunk's t_w): if k of them are
    // here, the k-th is among them and no chunk hides a key of the top k
    const uint32_t lo = t3[1];
    ovs = t3[2];
    if (E <= FIN_ENT - 64) {
      // group bases: an exclusive scan of the 256 group counts (wave 0, 4 a lane)
      if (wv == 0) {
        const v4i c4 = reinterpret_cast<const v4i*>(gcnt)[lane];
        const int t = c4[0] + c4[1] + c4[2] + c4[3];
        const int b = wave_incl_scan(t) - t;
        reinterpret_cast<v4i*>(gbase)[lane] = v4i{b, b + c4[0], b + c4[0] + c4[1], b + c4[0] + c4[1] + c4[2]};
      }
      __syncthreads();
      if (cap > 64) gather_candidates<2>(erow, wact, cnt8, gbase, FK, FP);
      else gather_candidates<1>(erow, wact, cnt8, gbase, FK, FP);
      __syncthreads();
      if (ovs == 0) {
        int got = -1;
        done = select_emit<32, false>(FK, FP, E, lo, k, hist, misc, out, &got);
        if (done && got != k && tid == 0) raise_error(ws, IDX_DERR_SELECT);
      }
      if (!done && nr <= BITMAP_KEYS) done = rare_select(ws, nr, k, wact, E, C, rs, FK, FP, bm, hist, misc, out);
    }
  }
  if (!done) {
    // ---- exact multi-pass select over the row's scores in memory
    __syncthreads();
    global_select_row(srow, nr, k, out, hist, misc);
  }
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
  uint64_t off_meta, off_ent, total;
  int meta_stride, ent_stride;
};

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

WsLayout layout_for(int rows, int max_keys) {
  const Plan a = plan_score(max_keys), b = plan_topk(max_keys);
  const int stride = (a.wg > b.wg ? a.wg : b.wg);
  WsLayout L;
  L.meta_stride = stride;
  L.ent_stride = stride < 4 * NT ? stride : 4 * NT;
  L.off_meta = WS_HDR;
  L.off_ent = align256(L.off_meta + (uint64_t)rows * stride * 8);
  L.total = align256(L.off_ent + (uint64_t)rows * L.ent_stride * CAP_MAX * 8);
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
  for (int j = 0; j < p->num_req; j++) {
    const int32_t r = p->req_indptr[j + 1] - p->req_indptr[j];
    if (r < 1) return IDX_EINVAL;
    if (r > IDX_GROUP_ROWS) return IDX_EUNSUPPORTED;
  }
  if (p->num_pages < 1 || p->max_pages < 1 || p->max_keys < 0) return IDX_EINVAL;
  if (p->req_max_keys)
    for (int j = 0; j < p->num_req; j++)
      if (p->req_max_keys[j] < 0 || p->req_max_keys[j] > p->max_keys) return IDX_EINVAL;
  if ((int64_t)p->max_keys > (int64_t)p->max_pages * IDX_PAGE_SIZE) return IDX_EINVAL;
  if (p->max_keys > (1 << 30)) return IDX_EUNSUPPORTED;
  if (check_ptr(p->q, 16) || check_ptr(p->w, 4) || check_ptr(p->k_cache, 16) || check_ptr(p->k_scale, 16) ||
      check_ptr(p->page_table, 4) || check_ptr(p->n_keys, 4))
    return IDX_EINVAL;
  return IDX_OK;
}

constexpr int SCORE_LDS = L_SCORE_END;
constexpr int SELECT_LDS = L_FIN_END;

int set_attrs() {
  if (g_attr_done) return IDX_OK;
  const void* fs[5] = {(const void*)score_kernel<1>, (const void*)score_kernel<2>, (const void*)score_kernel<4>,
                       (const void*)score_kernel<8>, (const void*)select_kernel};
  for (int i = 0; i < 5; i++) {
    const hipError_t e =
        hipFuncSetAttribute(fs[i], hipFuncAttributeMaxDynamicSharedMemorySize, i < 4 ? SCORE_LDS : SELECT_LDS);
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
    switch (P) {
      case 1: hipLaunchKernelGGL(score_kernel<1>, grid, dim3(NT), SCORE_LDS, st, args); break;
      case 2: hipLaunchKernelGGL(score_kernel<2>, grid, dim3(NT), SCORE_LDS, st, args); break;
      case 4: hipLaunchKernelGGL(score_kernel<4>, grid, dim3(NT), SCORE_LDS, st, args); break;
      default: hipLaunchKernelGGL(score_kernel<8>, grid, dim3(NT), SCORE_LDS, st, args); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  if (select_launch) {
    hipLaunchKernelGGL(select_kernel, dim3(IDX_GROUP_ROWS, grid.y), dim3(NT), SELECT_LDS, st, args);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  return IDX_OK;
}

void fill_common(KArgs& args, const WsLayout& L, void* ws) {
  args.ws = static_cast<uint8_t*>(ws);
  args.meta_stride = L.meta_stride;
  args.ent_stride = L.ent_stride;
  args.off_meta = L.off_meta;
  args.off_ent = L.off_ent;
}

int run_problem(const idx_problem* p, int32_t k, float* scores, int64_t ld, int32_t* topk, void* ws,
                size_t ws_bytes, void* stream, bool select) {
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
  args.ld = ld;
  args.rows = p->rows;
  args.max_pages = p->max_pages;
  args.max_keys = p->max_keys;
  args.num_pages = p->num_pages;
  args.k = k;
  args.chunk = pl.chunk;
  args.chunk_shift = 31 - __builtin_clz((unsigned)pl.chunk);
  args.mode = select ? (MODE_SCORE | MODE_PUBLISH) : MODE_SCORE;
  fill_common(args, L, ws);
  for (int j = 0; j < p->num_req; j++) {
    args.grp[j] = (uint32_t)p->req_indptr[j] | ((uint32_t)(p->req_indptr[j + 1] - p->req_indptr[j]) << 24);
    const int bound = p->req_max_keys ? p->req_max_keys[j] : p->max_keys;
    args.gmax[j] = bound;
  }
  return launch(args, pl.pages_per_wg, dim3(pl.wg, p->num_req), true, select, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int idx_abi_version(void) { return IDX_ABI_VERSION; }

int idx_workspace_bytes(int32_t rows, int32_t max_keys, int32_t k, size_t* bytes) {
  if (!bytes || rows < 1 || rows > (1 << 24) - 1 || max_keys < 0 || max_keys > (1 << 30) || k < 1 || k > IDX_KMAX)
    return IDX_EINVAL;
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
  return run_problem(p, 1, scores, ld_scores, nullptr, ws, ws_bytes, stream, false);
}

int idx_score_topk(const idx_problem* p, int32_t k, float* scores, int64_t ld_scores, int32_t* topk, void* ws,
                   size_t ws_bytes, void* stream) {
  return run_problem(p, k, scores, ld_scores, topk, ws, ws_bytes, stream, true);
}

int idx_topk(const float* scores, int64_t ld_scores, const int32_t* n_keys, int32_t rows, int32_t max_keys,
             int32_t k, int32_t* topk, void* ws, size_t ws_bytes, void* stream) {
  if (!scores || !n_keys || !topk || rows < 1 || rows > (1 << 24) - 1 || max_keys < 0 || max_keys > (1 << 30))
    return IDX_EINVAL;
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
    default: return "unknown error code";
  }
}

const char* idx_last_hip_error(void) { return g_hip_err; }

}  // extern "C"
