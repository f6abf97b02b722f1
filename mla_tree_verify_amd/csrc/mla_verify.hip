// MLA tree-verify attention for MI355X (gfx950): kernels and the C ABI.
//
// What is computed is stated in include/mla_verify.h. The method follows the
// pages' flash-decode design (page "The Decisive Microbench", section "The
// KV-Split Solution": each workgroup attends over one contiguous KV slice,
// writes its partial result with its log-sum-exp, and a light second kernel
// merges the slices) and their tile reuse across heads (page "The Flash
// Attention Kernel That Had to Be Built", section "The Final Architecture":
// one KV tile in shared memory serves several heads). The execution layout is
// designed for CDNA4 rather than taken from the pages' sm_120 kernels:
//
//  * One workgroup = one row block (64 consecutive (token, head) rows of the
//    [q, H] layout) x one KV chunk. Because the latent KV is shared by every
//    head, scores and values are dense contractions: S^T[keys x rows] =
//    K[keys x 576] Q^T and O^T[dims x rows] += V^T[dims x keys] P^T, both on
//    bf16 MFMA 32x32x16 with fp32 accumulation.
//  * 4 waves = 2 row halves x 2 dim halves, one wave per SIMD. A wave keeps
//    the queries of its 32 rows over its half of the 576 dims in registers
//    (72 VGPRs) and computes partial scores for every 32-key tile; each wave
//    owns half of a tile's keys, receives the partner's partial scores of
//    them through LDS, turns the full scores into weights, and the two waves
//    swap weights. Each then accumulates 256 of the 512 output dims of its
//    rows (128 AGPRs).
//  * KV tiles (and the block's query rows, once) go from HBM straight into
//    LDS with 16-byte buffer loads (buffer_load_dwordx4 ... lds) into a
//    4-slot ring loaded three tiles ahead; loads past the chunk or sequence
//    end return zeros. 16-byte chunks are XOR swizzled per key so that the
//    128-bit score-operand reads and the transposing value-operand reads
//    (ds_read_b64_tr_b16) avoid most bank conflicts.
//  * The S^T accumulator layout equals the P^T operand layout of the value
//    product, so softmax weights leave registers only for the swap. The next
//    tile's score MFMAs are issued before this tile's softmax so the two
//    overlap.
//  * The softmax reference max is fixed by the first visible tile and never
//    moves, so the accumulator is never rescaled inside the loop (weights may
//    reach 2^96; a chunk whose scores climb beyond that is redone once with
//    the chunk's own max).
//  * Softmax weights enter the value product as a bf16 hi+lo pair (two MFMAs
//    sharing the V operand), about 16 significant bits; a single bf16 weight
//    is an option.
//  * Workgroup ids are mapped so that consecutive ids on one XCD (ids are
//    dealt round-robin over the 8 XCDs) take the row blocks of one KV chunk,
//    so a chunk is read from HBM into one XCD's L2 and reused there (a chunk
//    whose row blocks straddle two XCDs is read by both).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "mla_verify.h"

#define LDS_AS __attribute__((address_space(3)))

namespace mlav {

constexpr int kRows = MLAV_ROWS;  // (token, head) rows per workgroup
constexpr int kDl = MLAV_DL;
constexpr int kDr = MLAV_DR;
constexpr int kTile = 32;                        // keys per wave tile
constexpr int kLatBytes = kTile * kDl * 2;       // 32768
constexpr int kRopeBytes = kTile * kDr * 2;      // 4096
constexpr int kTileBytes = kLatBytes + kRopeBytes;  // 36864
constexpr int kRing = 4;                         // tile slots: values, scores, two loading
constexpr int kXchgBytes = 4 * 2 * 64 * 16;      // one exchange area: [4 waves][2 chunks][64 lanes][16 B]
constexpr int kLdsBytes = kRing * kTileBytes + 2 * kXchgBytes;  // 163840 = all of a CU's LDS
constexpr int kThreads = 256;
static_assert(kRing * 128 == kDl && 128 * 4 * kRows <= kTileBytes,
              "the epilogue stages 128 output dims of all 64 rows in each ring slot");
static_assert(kLdsBytes <= 163840, "LDS per workgroup");
static_assert(32 * (kDl + kDr) * 2 == kTileBytes, "32 query rows fill one ring slot in the tile layout");
static_assert(32 * kDl * 2 <= kTileBytes, "the int16 epilogue stages 32 rows per ring slot");
constexpr int kXcds = 8;
constexpr int64_t kChunkGran = kTile;
// Smallest chunk the planner picks by itself: two tiles. Below that the
// per-workgroup fixed cost outweighs the extra CUs (at prefix 256, q 9:
// 64-key chunks 13.5 us per call, 32-key 13.4 us, 128-key 15.1 us; at
// prefix 512 64-key chunks beat 32-key ones).
constexpr int64_t kMinChunk = 64;
// Reference max placement, log2 units: the reference sits kRefShift above
// the first tile's max, so that tile's largest weight is 2^-32 and weights
// may grow to 2^96 (scores up to 128 above that max) before a redo; keys more
// than 94 below the max underflow to 0, a relative contribution below 2^-94.
// With weights at most 2^96, the accumulators stay finite while
// (keys in the chunk) x max|value| < 2^32.
constexpr float kRefShift = 32.0f;
constexpr float kRefHeadroom = 96.0f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct Args {
  const uint16_t* qn;    // [B, q, H, 512]
  const uint16_t* qr;    // [B, q, H, 64]
  const uint16_t* lat;   // [total, 512]
  const uint16_t* rope;  // [total, 64]
  const int32_t* parent; // [B, q]
  const int64_t* offs;   // [B + 1] or null (one sequence of single_n rows)
  const int32_t* idx;    // paged KV: [total] logical row -> row of the lat/rope pool; null = contiguous
  int64_t pool_rows;     // paged KV: rows of the pool
  float* out;            // [B, q, H, 512]
  float* lse;            // [B, q, H]
  // split partials, over [B, S, nrb * 64] rows (each sequence's q * H rows padded to whole row blocks)
  float* part_o;         // [B, S, nrb * 64, 512] fp32 partials
  int16_t* part_q;       // [B, S, nrb] blocks of 64 KB: int16 x part_scale, pair-major (compact_byte_off)
  float* part_scale;     // [B, S, nrb * 64]
  float* part_lse;       // [B, S, nrb * 64]
  unsigned long long* tickets;  // merge in the split kernel: [B, nrb] (epoch << 16 | arrivals)
  unsigned long long epoch;     // this call's ticket epoch (48 bits, not 0)
  int64_t single_n;
  int64_t total_kv;
  int64_t max_kv;
  int64_t chunk;
  float scale_log2;
  int32_t q;
  int32_t heads;         // query heads per token
  int32_t nrb;           // row blocks per sequence: ceil(q * heads / 64)
  int32_t batch;
  int32_t nsplit;
  int32_t nwork;
  int32_t per_xcd;
  int32_t fixed_ns;      // combine only: >0 forces every row's split count
  int32_t list_run;      // >0: batched chunk list dealt to the XCDs in runs of this many items
};

// ---------------------------------------------------------------------------
// shared device helpers
// ---------------------------------------------------------------------------
__device__ inline bool seq_bounds(const Args& a, int b, int64_t& row0, int64_t& n) {
  if (a.offs == nullptr) {
    row0 = 0;
    n = a.single_n;
    return true;
  }
  row0 = a.offs[b];
  const int64_t r1 = a.offs[b + 1];
  n = r1 - row0;
  return row0 >= 0 && r1 <= a.total_kv && n >= a.q && n <= a.max_kv;
}

// Ancestor-or-self mask of draft token t (bit u set = tree node u visible).
// The walk is bounded by q steps and by the index range, whatever the tree.
__device__ inline uint64_t ancestor_mask(const int32_t* parent, int q, int t) {
  uint64_t anc = 0;
  int node = t;
  for (int step = 0; step < q && node >= 0 && node < q; ++step) {
    anc |= 1ull << node;
    node = parent[node];
  }
  return anc;
}

// The same mask from a wave-held copy of the tree: lane u holds parent[u]
// (u < q). t is wave-uniform, so every step is a scalar read of one lane.
__device__ inline uint64_t ancestor_mask_wave(int par_lane, int q, int t) {
  uint64_t anc = 0;
  int node = t;
  for (int step = 0; step < q && node >= 0 && node < q; ++step) {
    anc |= 1ull << node;
    node = __builtin_amdgcn_readlane(par_lane, node);
  }
  return anc;
}

// The same mask for a per-lane token t (rows of several tokens share a
// wave): lane u holds parent[u] (u < q); each step fetches the parent of the
// lane's current node from the lane that holds it. q steps for every lane.
__device__ inline uint64_t ancestor_mask_lanes(int par_lane, int q, int t) {
  uint64_t anc = 0;
  int node = t;
  for (int step = 0; step < q; ++step) {
    const bool ok = node >= 0 && node < q;
    anc |= ok ? 1ull << node : 0ull;
    const int up = __shfl(par_lane, ok ? node : 0, 64);
    node = ok ? up : -1;
  }
  return anc;
}

__device__ inline bool key_visible(int64_t j, int64_t c1, int64_t prefix, uint64_t anc) {
  return j < c1 && (j < prefix || ((anc >> (j - prefix)) & 1ull));
}

// Visibility of the 32 keys [key0, key0 + 32) for one draft token, as a bit
// mask (bit k: key key0 + k). Keys below `prefix` are the cached prefix; key
// prefix + u is tree node u, visible when bit u of `anc` is set; keys at or
// past c1 (the chunk end) are not part of this chunk. All operands are
// wave-uniform, so this is scalar work.
__device__ inline uint32_t tile_visibility(int64_t key0, int64_t c1, int64_t prefix, uint64_t anc) {
  const int64_t np = prefix - key0;  // tile keys inside the prefix
  uint32_t m;
  if (np >= 32) {
    m = 0xffffffffu;
  } else {
    m = np > 0 ? ((1u << np) - 1u) : 0u;
    const int64_t sh = key0 - prefix;  // tree node at bit 0 (negative: inside the prefix)
    uint64_t tm;
    if (sh >= 0)
      tm = sh < 64 ? (anc >> sh) : 0ull;
    else
      tm = -sh < 64 ? (anc << -sh) : 0ull;
    m |= (uint32_t)tm;
  }
  const int64_t nv = c1 - key0;  // tile keys before the chunk end
  if (nv < 32) m &= nv > 0 ? ((1u << nv) - 1u) : 0u;
  return m;
}

// Logical <-> physical 16-byte chunk swizzles (XOR on the chunk index).
// Latent rows (64 chunks): the low 4 bits. The LDS has 64 four-byte banks,
// i.e. 16 chunk positions: the 128-bit score-operand reads of 16 consecutive
// keys at one logical chunk then hit 16 different positions, and the
// transposing value-operand reads (4 consecutive keys x 2 adjacent chunks
// per 16 lanes) hit 8 different pairs.
__device__ inline int swz(int k) { return ((k & 3) << 1) | ((k >> 2) & 1) | (k & 8); }
// Rope rows (8 chunks, 128 B, two rows per 16 positions): 16 consecutive keys
// at one logical chunk hit 16 different positions.
__device__ inline int swz_rope(int k) { return (k >> 1) & 7; }

__device__ inline float fmax3(float a, float b) { return __builtin_fmaxf(a, b); }

// max(m, |a|, |b|) in one v_max3_f32 with abs modifiers. Written out because
// for values read from accumulator registers the compiler emitted two-input
// maxes plus canonicalising moves (about 3.6 instructions per value instead
// of 0.5).
__device__ inline float max3_abs(float m, float a, float b) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

__device__ inline float partner_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax3(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float partner_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int kCtrl>
__device__ inline float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}

// Maximum over the 64 lanes of a wave, returned in every lane: quad_perm
// steps within quads, mirrors within rows of 16, then the row-pair and
// wave-half swaps.
__device__ inline float wave_max(float x) {
  x = fmax3(x, dpp_f32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmax3(x, dpp_f32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmax3(x, dpp_f32<0x141>(x));  // row_half_mirror
  x = fmax3(x, dpp_f32<0x140>(x));  // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmax3(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return partner_max(x);
}

// Maximum / sum over the 16 lanes of each row of a wave, in every lane of the
// row; the 32-lane forms add the row-pair swap (lanes 0..31 and 32..63).
__device__ inline float row16_max(float x) {
  x = fmax3(x, dpp_f32<0xB1>(x));
  x = fmax3(x, dpp_f32<0x4E>(x));
  x = fmax3(x, dpp_f32<0x141>(x));
  return fmax3(x, dpp_f32<0x140>(x));
}
__device__ inline float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  return x + dpp_f32<0x140>(x);
}
__device__ inline float half32_max(float x) {
  x = row16_max(x);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax3(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half32_sum(float x) {
  x = row16_sum(x);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Work id -> (sequence, split, row block); the row blocks of one chunk are consecutive ids.
// Values are made wave-uniform explicitly so that addresses built from them
// stay in scalar registers.
__device__ inline bool decode_work(const Args& a, int& b, int& s, int& t) {
  const int bid = blockIdx.x;
  const int w = uniform((bid % kXcds) * a.per_xcd + bid / kXcds);
  if (w >= a.nwork) return false;
  t = uniform(w % a.nrb);
  const int bs = uniform(w / a.nrb);
  s = uniform(bs % a.nsplit);
  b = uniform(bs / a.nsplit);
  return true;
}

// Batched calls: the chunks of every sequence form one list, in this order:
//   1. one entry per sequence whose offsets are inconsistent (its NaN rows),
//   2. every full chunk (`chunk` keys), by sequence, then split,
//   3. each sequence's last, shorter chunk; up to 64 sequences longest first
//      (16 length classes of chunk / 16 keys, each class in sequence order),
//      beyond that in sequence order,
// so that the long work starts first and the short tail chunks fill the CUs
// at the end (an XCD hands its workgroups to its CUs in id order). Item i of
// the list is row block i % nrb of chunk i / nrb. The dispatcher sends
// workgroup id w to XCD w % 8; ids map to items so that each XCD takes runs
// of list_run consecutive items (row blocks of one chunk, sharing its KV in
// that XCD's L2), the runs dealt over the XCDs in rounds of 8, every other
// round in reverse order (the longest runs do not all land on the same XCDs).
// Every wave computes the same (uniform) result from the offsets, one
// sequence per lane.

// One sequence per lane: bounds check, full chunks and the length class of
// the last, shorter chunk (-1: none).
__device__ inline void list_lane(const Args& a, int sb, bool& ok, int64_t& r0, int& len, int& f, int& cls) {
  ok = false;
  r0 = 0;
  len = 0;
  f = 0;
  cls = -1;
  if (sb < a.batch) {
    r0 = a.offs[sb];
    const int64_t r1 = a.offs[sb + 1];
    const int64_t n = r1 - r0;
    ok = r0 >= 0 && r1 <= a.total_kv && n >= a.q && n <= a.max_kv;
    if (ok) {
      const uint32_t c = (uint32_t)a.chunk;  // chunk and n are at most MLAV_MAX_KV
      len = (int)n;
      f = (int)((uint32_t)len / c);
      const uint32_t rem = (uint32_t)len - (uint32_t)f * c;
      cls = rem > 0 ? (int)(rem * 16u / c) : -1;
    }
  }
}

__device__ inline int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Lanes of m below this lane.
__device__ inline int mask_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ inline int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ inline int64_t readlane_i64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Work id -> (sequence, split, row block) through the chunk list, with the
// sequence's first row and length; ok = false for an inconsistent sequence
// (split 0: write its NaN rows). False past the list's end.
__device__ inline bool decode_list(const Args& a, int& b, int& s, int& t, int64_t& row0, int64_t& n, bool& ok) {
  const int bid = blockIdx.x;
  const int g = a.list_run;
  const int j = bid / kXcds;  // the j-th workgroup dispatched on XCD bid % 8
  const int rnd = j / g;      // round of runs: run rnd * 8 + x goes to XCD x, reversed every other round
  const int x = (rnd & 1) ? kXcds - 1 - bid % kXcds : bid % kXcds;
  const int item = uniform((rnd * kXcds + x) * g + j % g);
  int k = uniform(item / a.nrb);  // list entry
  t = uniform(item % a.nrb);
  const int lane = threadIdx.x & 63;
  const int B = a.batch;
  bool lok;
  int64_t lr0;
  int llen, lf, lcls;
  // sets the outputs from lane L of the current group
  auto take = [&](int g0, int L, int split, bool valid) {
    b = g0 + L;
    s = split;
    ok = valid;
    row0 = valid ? readlane_i64(lr0, L) : 0;
    n = valid ? readlane_i(llen, L) : 0;
  };
  if (B <= 64) {
    list_lane(a, lane, lok, lr0, llen, lf, lcls);
    const uint64_t inv = __ballot(lane < B && !lok);
    const int ninv = __popcll(inv);
    if (k < ninv) {
      take(0, __builtin_ctzll(__ballot(lane < B && !lok && mask_rank(inv) == k)), 0, false);
      return true;
    }
    k -= ninv;
    const int incl = wave_incl_scan(lf, lane);
    const int nfull = readlane_i(incl, 63);
    if (k < nfull) {
      const int L = __builtin_ctzll(__ballot(incl > k));
      take(0, L, k - (readlane_i(incl, L) - readlane_i(lf, L)), true);
      return true;
    }
    k -= nfull;
    // rank of each lane's last chunk: longer classes first, then sequence order
    int pos = -1, base = 0;
#pragma unroll
    for (int c = 15; c >= 0; --c) {
      const uint64_t m = __ballot(lcls == c);
      if (lcls == c) pos = base + mask_rank(m);
      base += __popcll(m);
    }
    if (k >= base) return false;
    const int L = __builtin_ctzll(__ballot(pos == k));
    take(0, L, readlane_i(lf, L), true);
    return true;
  }
  // more than 64 sequences: section sizes first, then the search
  int ninv = 0, nfull = 0, npart = 0;
  for (int g0 = 0; g0 < B; g0 += 64) {
    list_lane(a, g0 + lane, lok, lr0, llen, lf, lcls);
    ninv += __popcll(__ballot(g0 + lane < B && !lok));
    nfull += readlane_i(wave_incl_scan(lf, lane), 63);
    npart += __popcll(__ballot(lcls >= 0));
  }
  const int sec = k < ninv ? 0 : k < ninv + nfull ? 1 : k < ninv + nfull + npart ? 2 : -1;
  if (sec < 0) return false;
  int rank = sec == 0 ? k : sec == 1 ? k - ninv : k - ninv - nfull;
  for (int g0 = 0; g0 < B; g0 += 64) {
    list_lane(a, g0 + lane, lok, lr0, llen, lf, lcls);
    if (sec == 1) {
      const int incl = wave_incl_scan(lf, lane);
      const int tot = readlane_i(incl, 63);
      if (rank < tot) {
        const int L = __builtin_ctzll(__ballot(incl > rank));
        take(g0, L, rank - (readlane_i(incl, L) - readlane_i(lf, L)), true);
        return true;
      }
      rank -= tot;
    } else {
      const bool mine = sec == 0 ? (g0 + lane < B && !lok) : (lcls >= 0);
      const uint64_t m = __ballot(mine);
      if (rank < (int)__popcll(m)) {
        const int L = __builtin_ctzll(__ballot(mine && mask_rank(m) == rank));
        take(g0, L, sec == 0 ? 0 : readlane_i(lf, L), sec != 0);
        return true;
      }
      rank -= __popcll(m);
    }
  }
  return false;
}

// NaN into the output rows of row block rbk of sequence b (inconsistent offsets).
__device__ inline void write_nan_rows(const Args& a, int b, int rbk, int tid, int nthreads) {
  const float nan = __builtin_nanf("");
  const int64_t rows_seq = (int64_t)a.q * a.heads;
  const int64_t r0 = (int64_t)rbk * kRows;
  const int nr = (int)(rows_seq - r0 < kRows ? rows_seq - r0 : kRows);
  float* o = a.out + ((int64_t)b * rows_seq + r0) * kDl;
  for (int i = tid; i < nr * kDl; i += nthreads) o[i] = nan;
  for (int i = tid; i < nr; i += nthreads) a.lse[(int64_t)b * rows_seq + r0 + i] = nan;
}

// ---------------------------------------------------------------------------
// split kernel: bf16 MFMA
// ---------------------------------------------------------------------------
// Buffer descriptor over `bytes` bytes at `base` (gfx9 raw buffer, stride 0):
// loads past `bytes` return zeros, which zero-fills tiles past the sequence end.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Issue this wave's quarter of the direct-to-LDS loads of one 32-key tile
// (issue_tile_part: load `part` of the nine).
// key_rel = first key of the tile relative to the descriptors' first row.
// Latent row k lands at buf + 1024 k with its 16-byte chunks XOR-swizzled by
// swz(k); the rope rows follow the 32 latent rows, 128 B each, swizzled by
// swz_rope(k).
// key_rel = kNoTile requests nothing: the byte offset is then set past any
// descriptor range (at most 4e6 rows x 1 KB, below 2^32), so the load fills
// the slot with zeros without reading memory (callers use it to keep the
// number of loads per step constant).
constexpr int kNoTile = -1;
constexpr uint32_t kOutOfRange = 0xFFFFF000u;
__device__ inline void issue_tile_part(LDS_AS char* buf, __amdgpu_buffer_rsrc_t lat_rs,
                                       __amdgpu_buffer_rsrc_t rope_rs, int key_rel, int wave, int lane,
                                       int rope_voff, int part) {
  // The whole byte offset goes in the VGPR operand: raw-buffer range checks
  // cover the VGPR offset (plus the immediate) but not the SGPR offset.
  const bool none = key_rel < 0;
  if (part < 8) {
    const int k = 4 * part + wave;
    const uint32_t off = (uint32_t)(key_rel + k) * 1024u + 16u * (uint32_t)(lane ^ swz(k));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(lat_rs, (LDS_AS void*)(buf + k * 1024), 16,
                                             (int)(none ? kOutOfRange : off), 0, 0, 0);
  } else {
    const uint32_t off = (uint32_t)(key_rel + 8 * wave) * 128u + (uint32_t)rope_voff;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rope_rs, (LDS_AS void*)(buf + kLatBytes + wave * 1024), 16,
                                             (int)(none ? kOutOfRange : off), 0, 0, 0);
  }
}

__device__ inline void issue_tile(LDS_AS char* buf, __amdgpu_buffer_rsrc_t lat_rs,
                                  __amdgpu_buffer_rsrc_t rope_rs, int key_rel, int wave, int lane,
                                  int rope_voff) {
#pragma unroll
  for (int part = 0; part < 9; ++part)
    issue_tile_part(buf, lat_rs, rope_rs, key_rel, wave, lane, rope_voff, part);
}

// Paged KV (one token per page): the same tile layout, gathered through a
// page table. idx_lane holds, in lane j < 32, the pool row of key j of the
// tile (-1: none, the slot gets zeros); rope_idx is the pool row of this
// lane's rope row 8 wave + (lane>>3). A latent row is one whole instruction,
// so its pool row is wave-uniform (readlane); the descriptors span the pool
// and a row outside it reads zeros.
__device__ inline void issue_tile_part_paged(LDS_AS char* buf, __amdgpu_buffer_rsrc_t lat_rs,
                                             __amdgpu_buffer_rsrc_t rope_rs, int idx_lane, int rope_idx,
                                             int wave, int lane, int rope_loff, int part) {
  if (part < 8) {
    const int k = 4 * part + wave;
    const int prow = __builtin_amdgcn_readlane(idx_lane, k);
    const uint32_t off = prow >= 0 ? (uint32_t)prow * 1024u + 16u * (uint32_t)(lane ^ swz(k)) : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(lat_rs, (LDS_AS void*)(buf + k * 1024), 16, (int)off, 0, 0, 0);
  } else {
    const uint32_t off = rope_idx >= 0 ? (uint32_t)rope_idx * 128u + (uint32_t)rope_loff : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rope_rs, (LDS_AS void*)(buf + kLatBytes + wave * 1024), 16,
                                             (int)off, 0, 0, 0);
  }
}

// Lane bases of the K operand reads. Score k-step ks of a wave reads 16-byte
// chunk c = 36 kDh + 2 ks + (lane>>5) of key lane&31's 576-d row (chunks
// 0..63 latent, 64..71 rope). A latent chunk is stored at position
// (c & ~15) | ((c & 15) ^ swz(key)); since 36 kDh + 2 ks is even, that is
// (c & ~15) | (e2 ^ hs) with e2 = (36 kDh + 2 ks) & 15 and
// hs = (lane>>5) ^ swz(key), so eight per-lane bases (one per e2) plus a
// compile-time offset cover the latent k-steps; rope chunk c - 64 is at
// position (c - 64) ^ swz_rope(key), four bases.
struct KBases {
  int lat[8];   // key * 1024 + 16 * ((2e) ^ hs)
  int rope[4];  // kLatBytes + key * 128 + 16 * ((2e) ^ ((lane>>5) ^ swz_rope(key)))
};

__device__ inline KBases make_kbases(int key, int half) {
  KBases kb;
  const int hs = half ^ swz(key);
  const int hr = half ^ swz_rope(key);
#pragma unroll
  for (int e = 0; e < 8; ++e) kb.lat[e] = key * 1024 + 16 * ((2 * e) ^ hs);
#pragma unroll
  for (int e = 0; e < 4; ++e) kb.rope[e] = kLatBytes + key * 128 + 16 * ((2 * e) ^ hr);
  return kb;
}

// Byte offset (within a ring slot) of this lane's K operand for k-step ks.
template <int kDh>
__device__ inline int k_frag_off(const KBases& kb, int ks) {
  const int c0 = 36 * kDh + 2 * ks;  // even chunk index of the pair
  if (c0 < 64) return kb.lat[(c0 & 15) >> 1] + 16 * (c0 & ~15);
  return kb.rope[(c0 - 64) >> 1];
}

__device__ inline bf16x8_t lds_b128(const LDS_AS char* p) { return *(const LDS_AS bf16x8_t*)p; }

// Workgroup barrier for LDS exchanges: this wave's LDS reads and writes are
// complete (lgkmcnt(0)) and every wave has arrived. Unlike __syncthreads(),
// it does not wait for outstanding tile loads (that workgroup-scope fence
// waits vmcnt(0), which would serialise the loads three steps ahead); tile
// loads are waited for explicitly with vmcnt. The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt: no wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Returns x unchanged but opaque to the optimiser, so that an address formed
// once per loop iteration is not split into one hoisted register per use.
__device__ inline int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Partial scores of one tile over this wave's half of the 576 dims:
// S^T[32 keys x 32 rows] = K[32 keys x 288] Q^T[288 x 32 rows] (a row is one
// (token, head) pair).
template <int kDh>
__device__ inline f32x16_t tile_scores(const LDS_AS char* buf, const bf16x8_t (&qreg)[18],
                                       const KBases& kb) {
  f32x16_t sc = {};
#pragma unroll
  for (int ks = 0; ks < 18; ++ks)
    sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(buf + k_frag_off<kDh>(kb, ks)), qreg[ks], sc,
                                                 0, 0, 0);
  return sc;
}

// One workgroup = one row block (64 consecutive (token, head) rows) x one KV
// chunk; 4 waves = 2 row halves (hh) x 2 dim halves (kDh). Both waves of a
// row half compute partial scores of every tile over their dim half. The
// softmax is split between them: the wave with dim half kDh owns the tile's keys
// [16 kDh, 16 kDh + 16) (accumulator elements r = 8 kDh .. 8 kDh + 7), so
// each wave sends its partner the partial scores of the partner's keys,
// turns the full scores of its own keys into bf16 hi + lo weights, and the
// two swap those weights. Each wave then accumulates 256 of the 512 output
// dims over all 32 keys.
//
// LDS: four ring slots (separate objects, so the compiler can see that a
// tile load into one slot does not write the slots being read and issues no
// wait for it), an 8 KB partial-score exchange and an 8 KB weight exchange:
// 163840 bytes. A tile is loaded three steps ahead of its value product.
// Merge in the split kernel (plans of 2..4 splits): every workgroup of a row
// block writes its partial rows with device-coherent stores (sc1: written
// through the XCD's L2, whose lines other XCDs do not see), waits until they
// are performed and takes a ticket; the one that takes the last ticket reads
// the block's rows with device-coherent loads and merges them, so no combine
// launch follows. A full release/acquire fence pair would instead write back
// and invalidate the whole L2 of the XCD, which costs more than the merge.
// A ticket word is (epoch << 16) | arrivals; a word from another epoch (a
// previous call, or whatever the workspace held) counts as empty, and the
// last arriver resets it to 0, so the workspace needs no clearing and a
// replayed graph (same epoch) starts from 0 each time.
constexpr int kMaxFusedSplits = 4;
constexpr int kCoherent = 16;  // buffer cache policy: sc1 (device scope)

// Compact partials of one row block (64 rows x 512 int16 values, 64 KB) lie
// pair-major: [32 pairs of 16 dims][64 rows][16 dims]. Byte offset of row h's
// 32 bytes of pair p within the block.
__device__ inline int compact_byte_off(int p, int h) { return (p * kRows + h) * 32; }
template <int kNs>
__device__ inline void merge_block(const Args& a, LDS_AS char* xs, int b, int rbk, int wave, int lane) {
  constexpr int ns = kNs;
  unsigned long long* tk = a.tickets + (int64_t)b * a.nrb + rbk;
  const int rows_seq = a.q * a.heads;
  const int64_t out_row0 = (int64_t)b * rows_seq + rbk * kRows;  // first output row of the block
  const int nvalid = rows_seq - rbk * kRows < kRows ? rows_seq - rbk * kRows : kRows;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's coherent partial stores are performed
  __syncthreads();                // (also: every wave is done with the exchange area)
  if (threadIdx.x == 0) {
    unsigned long long old = __hip_atomic_load(tk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int last = 0;
    for (int tries = 0; tries < 64; ++tries) {  // at most ns - 1 concurrent updates can make a CAS fail
      const unsigned long long nw = (old >> 16) == a.epoch ? old + 1 : (a.epoch << 16) | 1ull;
      const unsigned long long seen = atomicCAS(tk, old, nw);
      if (seen == old) {
        last = (int)(nw & 0xFFFFull) == ns;
        break;
      }
      old = seen;
    }
    *(LDS_AS int*)xs = last;
  }
  __syncthreads();
  if (*(const LDS_AS int*)xs == 0) return;
  // wave w merges pairs [8 w, 8 w + 8) of the block for all 64 rows: lane
  // (h & 31, half) takes row 32 rh + (lane & 31), dims 16 p + 8 half .. + 8,
  // for the 16 (pair, row half) units of the wave, kR units per round of loads
  // (all of a round in flight); each lane fetches its row's lse and scale of
  // every split
  const int sstride = a.nrb * kRows;
  const int64_t row_base = ((int64_t)b * a.nsplit * a.nrb + rbk) * kRows;  // split 0, row 0 of the block
  __amdgpu_buffer_rsrc_t rs[kNs];  // the block's 64 KB of each split
#pragma unroll
  for (int sp = 0; sp < kNs; ++sp)
    rs[sp] = make_rsrc(a.part_q + (row_base + (int64_t)sp * sstride) * kDl, kRows * kDl * 2);
  const int half = lane >> 5;
  constexpr int kR = 4;
#pragma unroll 1
  for (int u0 = 0; u0 < 16; u0 += kR) {
    u32x4_t qv[kR][kNs];
    float lz[kR][kNs], sc[kR][kNs];
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const int pr = 8 * wave + ((u0 + k) >> 1);
      const int h = 32 * ((u0 + k) & 1) + (lane & 31);
#pragma unroll
      for (int sp = 0; sp < kNs; ++sp) {
        qv[k][sp] = __builtin_amdgcn_raw_buffer_load_b128(rs[sp], compact_byte_off(pr, h) + 16 * half, 0, kCoherent);
        // lse (half 0) or scale (half 1) of the row; the lane halves swap below
        const int64_t rr = row_base + (int64_t)sp * sstride + h;
        lz[k][sp] = __hip_atomic_load((half ? a.part_scale : a.part_lse) + rr, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int k = 0; k < kR; ++k)
#pragma unroll
      for (int sp = 0; sp < kNs; ++sp) {
        const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(lz[k][sp]), __float_as_uint(lz[k][sp]),
                                                        false, false);
        lz[k][sp] = __uint_as_float(x[0]);
        sc[k][sp] = __uint_as_float(x[1]);
      }
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const int pr = 8 * wave + ((u0 + k) >> 1);
      const int h = 32 * ((u0 + k) & 1) + (lane & 31);
      float M = -INFINITY;
#pragma unroll
      for (int sp = 0; sp < kNs; ++sp) M = fmax3(M, lz[k][sp]);
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      float wsum = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int sp = 0; sp < kNs; ++sp) {
          const float w = __builtin_amdgcn_exp2f((lz[k][sp] - M) * kLog2e);  // 0 for a split that saw no key
          wsum += w;
          const float f = w * sc[k][sp];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int32_t v = (int32_t)qv[k][sp][e];
            acc[2 * e] += f * (float)((v << 16) >> 16);
            acc[2 * e + 1] += f * (float)(v >> 16);
          }
        }
      }
      if (h < nvalid) {
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
        float* o = a.out + (out_row0 + h) * kDl + 16 * pr + 8 * half;
        *(f32x4_t*)o = (f32x4_t){acc[0], acc[1], acc[2], acc[3]} * inv;
        *(f32x4_t*)(o + 4) = (f32x4_t){acc[4], acc[5], acc[6], acc[7]} * inv;
        if (pr == 0 && half == 0) a.lse[out_row0 + h] = wsum > 0.f ? M + __builtin_amdgcn_logf(wsum) * kLn2 : -INFINITY;
      }
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(tk, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int kDh, bool kHiLo, bool kCompact, bool kPaged, bool kFused>
__device__ inline void split_body(const Args& a, LDS_AS char* r0, LDS_AS char* r1, LDS_AS char* r2,
                                  LDS_AS char* r3, LDS_AS char* xs, LDS_AS char* xp, int b, int s,
                                  int rbk, int wave, int hh, int lane, int64_t row0, int64_t n) {
  constexpr int kOwn = 8 * kDh;         // this wave's softmax elements
  constexpr int kSend = 8 * (1 - kDh);  // the partner's
  const int half = lane >> 5;
  // sequence positions fit in 32 bits (a sequence has at most MLAV_MAX_KV rows)
  const int n32 = (int)n;
  const int chunk = (int)a.chunk;
  const int prefix = n32 - a.q;
  const int c0 = s * chunk;
  const int c1 = c0 + chunk < n32 ? c0 + chunk : n32;
  const int nsplit_b = (n32 + chunk - 1) / chunk;
  const int ntiles = (c1 - c0 + kTile - 1) / kTile;
  // This lane's row: row `head` of the block, (token, head) row r of the
  // sequence, r = token * heads + head index; rows past q * heads pad the last
  // block (their queries read as zeros; they take the last row's token for
  // the tree mask, and their results are never stored as outputs).
  const int head = 32 * hh + (lane & 31);
  const int rows_seq = a.q * a.heads;
  const int r_lane = rbk * kRows + head;
  const int r_src = r_lane < rows_seq ? r_lane : rows_seq - 1;
  const int tok = r_src / a.heads;

  // contiguous KV: descriptors over this chunk's rows onward; paged KV: over the pool
  const __amdgpu_buffer_rsrc_t lat_rs =
      kPaged ? make_rsrc(a.lat, (uint32_t)a.pool_rows * (kDl * 2))
             : make_rsrc(a.lat + (row0 + c0) * kDl, (uint32_t)(n32 - c0) * (kDl * 2));
  const __amdgpu_buffer_rsrc_t rope_rs =
      kPaged ? make_rsrc(a.rope, (uint32_t)a.pool_rows * (kDr * 2))
             : make_rsrc(a.rope + (row0 + c0) * kDr, (uint32_t)(n32 - c0) * (kDr * 2));
  // rope row 8 wave + (lane>>3) of a tile: LDS position lane&7 holds
  // logical chunk (lane&7) ^ swz_rope(row)
  const int rope_loff = 16 * ((lane & 7) ^ swz_rope(8 * wave + (lane >> 3)));
  const int rope_voff = (lane >> 3) * 128 + rope_loff;
  // every step issues nine loads (tiles past the chunk end request nothing)
  // so that vmcnt(9) always means "all but the latest tile landed"; paged KV
  // adds one page-table load per step (issued before the step's tile loads),
  // so its count is 10
  auto tile_rel = [&](int i) { return i < ntiles ? i * kTile : kNoTile; };
  // page-table entries of tile i: every lane loads from a valid address (so
  // this is exactly one load instruction); the raw entries are checked only
  // when used, a step later, so that nothing waits for the load early
  auto idx_valid = [&](int i) {
    const int L = c0 + i * kTile + (lane & 31);
    return lane < 32 && i < ntiles && L < c1;
  };
  auto load_idx = [&](int i) -> int {
    return a.idx[row0 + (idx_valid(i) ? c0 + i * kTile + (lane & 31) : c0)];
  };
  // lane j < 32: the pool row of key j of tile i, -1 past the chunk or outside the pool
  auto checked_idx = [&](int i, int raw) { return idx_valid(i) && raw >= 0 && raw < a.pool_rows ? raw : -1; };
  auto rope_rows = [&](int idx_lane) { return __shfl(idx_lane, 8 * wave + (lane >> 3), 64); };
  auto issue_paged = [&](LDS_AS char* buf, int idx_lane) {
    const int ri = rope_rows(idx_lane);
#pragma unroll
    for (int part = 0; part < 9; ++part)
      issue_tile_part_paged(buf, lat_rs, rope_rs, idx_lane, ri, wave, lane, rope_loff, part);
  };
  int idx_cur = -1;  // paged: raw page-table entries of the next tile to load
  // the first three tiles again, for the redo after a reference-max
  // overflow; paged KV reads their page-table entries first and the fourth
  // tile's between tiles 1 and 2 (the same ten loads as a step)
  auto restart_tiles = [&]() {
    if constexpr (kPaged) {
      const int i0 = load_idx(0), i1 = load_idx(1), i2 = load_idx(2);
      issue_paged(r0, checked_idx(0, i0));
      issue_paged(r1, checked_idx(1, i1));
      __builtin_amdgcn_sched_barrier(0);
      idx_cur = load_idx(3);
      __builtin_amdgcn_sched_barrier(0);
      issue_paged(r2, checked_idx(2, i2));
    } else {
      issue_tile(r0, lat_rs, rope_rs, 0, wave, lane, rope_voff);
      issue_tile(r1, lat_rs, rope_rs, tile_rel(1), wave, lane, rope_voff);
      issue_tile(r2, lat_rs, rope_rs, tile_rel(2), wave, lane, rope_voff);
    }
  };

  int par_lane;
  // resident queries for this wave's dim half: B operand of S^T = K Q^T
  bf16x8_t qreg[18];
  // The block's 64 query rows arrive like two key tiles (whole 1 KB rows per
  // load, where loading the operand layout directly would touch 32 rows per
  // load): rows 0..31 into ring slot 3, rows 32..63 into slot 2, both in the
  // tile layout, so that each wave reads its operand with the K-operand
  // pattern. Rows past the block's valid rows read as zeros. Tile 2 is
  // requested once every wave holds its queries (slot 2 free). Issue order:
  // tile 0, the parents, the queries, tile 1 (paged: the fourth tile's
  // page-table entries after it), so that one vmcnt covers tile 0 and the
  // queries.
  int idx2 = -1;  // paged: raw page-table entries of tile 2
  {
    int i1 = -1;
    if constexpr (kPaged) {
      const int i0 = load_idx(0);
      i1 = load_idx(1);
      idx2 = load_idx(2);
      issue_paged(r0, checked_idx(0, i0));
    } else {
      issue_tile(r0, lat_rs, rope_rs, 0, wave, lane, rope_voff);
    }
    __builtin_amdgcn_sched_barrier(0);
    par_lane = lane < a.q ? a.parent[(int64_t)b * a.q + lane] : -1;
    const int64_t qrow0 = (int64_t)b * rows_seq + rbk * kRows;
    const int qvalid = rows_seq - rbk * kRows < kRows ? rows_seq - rbk * kRows : kRows;
    const __amdgpu_buffer_rsrc_t qn_rs = make_rsrc(a.qn + qrow0 * kDl, (uint32_t)qvalid * (kDl * 2));
    const __amdgpu_buffer_rsrc_t qr_rs = make_rsrc(a.qr + qrow0 * kDr, (uint32_t)qvalid * (kDr * 2));
    issue_tile(r3, qn_rs, qr_rs, 0, wave, lane, rope_voff);
    issue_tile(r2, qn_rs, qr_rs, 32, wave, lane, rope_voff);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPaged) {
      issue_paged(r1, checked_idx(1, i1));
      __builtin_amdgcn_sched_barrier(0);
      idx_cur = load_idx(3);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      issue_tile(r1, lat_rs, rope_rs, tile_rel(1), wave, lane, rope_voff);
    }
  }

  // V^T operand (transposing reads): in each 16-lane group lane i reads 4
  // dims (16 dhalf + 4 (i&3) ..) of key row kk = 4 half + (i>>2) (+8 v for
  // the second read, +16 per key step); chunk 4 db + 2 dhalf + ((i&3)>>1) of
  // dim block db. Under swz(kk) the low chunk bits become
  // z0 ^ 4 (db & 1) ^ 8 (((db >> 1) ^ v) & 1), with z0 below, and db >> 2
  // adds 16 chunks: four per-lane bases vb[m], m = (db & 1) + 2 (((db >> 1) ^ v) & 1).
  int vb[4];
  {
    const int i = lane & 15;
    const int dhalf = (lane >> 4) & 1;
    const int kk = 4 * half + (i >> 2);
    const int z0 = (2 * dhalf + ((i & 3) >> 1)) ^ (((i >> 2) << 1) | half);
#pragma unroll
    for (int m = 0; m < 4; ++m) vb[m] = kk * 1024 + 16 * (z0 ^ (4 * m)) + 8 * (i & 1);
  }

  // a block of one token (heads a multiple of 64): the uniform walk; else per lane
  const uint64_t anc = a.heads % kRows == 0 ? ancestor_mask_wave(par_lane, a.q, uniform(tok))
                                            : ancestor_mask_lanes(par_lane, a.q, tok);

  const int partner = wave ^ 1;  // same head half, other dim half
  const KBases kb = make_kbases(lane & 31, half);
  // exchange areas: [wave][chunk][lane][16 B], 2 KB per wave
  LDS_AS char* xs_mine = xs + wave * 2048 + lane * 16;
  LDS_AS char* xs_part = xs + partner * 2048 + lane * 16;
  LDS_AS char* xp_mine = xp + wave * 2048 + lane * 16;
  LDS_AS char* xp_part = xp + partner * 2048 + lane * 16;
  // ring slot r (a compile-time r selects the object itself)
  auto ring = [&](int r) { return r == 0 ? r0 : (r == 1 ? r1 : (r == 2 ? r2 : r3)); };
  // lane holds keys 8*(r>>2) + 4*half + (r&3) of a tile in accumulator element r
  auto key_visible_bit = [&](uint32_t vis, int r) {
    return ((vis >> (4 * half + 8 * (r >> 2) + (r & 3))) & 1u) != 0;
  };

  // Online softmax with a reference max that never moves inside the loop:
  // the first tile with a visible key fixes it (kRefShift above the max of
  // that tile's full scores, the same in all four waves), later weights are
  // 2^(s - m_ref), exact for any m_ref. A score more than kRefHeadroom above
  // m_ref could overflow; then the chunk is redone once with m_ref = the
  // chunk's observed max, which no score exceeds. The accumulator is never
  // rescaled. (With the reference at the first tile's max and a headroom of
  // 2^64, keys scaled by 8 in 1 % of the rows made most workgroups redo their
  // chunk, and the slowest workgroup sets the kernel's time.)
  f32x16_t acc[8];
  float m_ref = -INFINITY;  // log2 units, this lane's head
  float l_run = 0.f;        // this lane's share of the softmax denominator (own keys)
  float m_seen = -INFINITY; // max over own keys
  bool have_ref = false;    // this lane's row has seen a visible key (fixed its m_ref)
  float acc_amax = 0.f;     // largest |accumulator| of this lane after the chunk
  // A chunk that starts inside the prefix gives every row a visible key in
  // its first tile, so all rows fix m_ref there. A chunk of tree keys only
  // (rows of several tokens can see different keys) may leave rows without a
  // reference after the first tile: its masked steps then exchange tile
  // maxima so that each such row fixes m_ref at its first visible tile.
  const bool ref_xchg = c0 >= prefix;  // uniform
  const float sl2 = a.scale_log2;  // > 0, so max(s) * sl2 = max(s * sl2)
  for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = (f32x16_t){};
    l_run = 0.f;
    int ovf = 0;

    // prologue: tiles 0..2 in flight; tile 0's partial scores exchanged in
    // full (through ring slot 3, free until tile 3 is loaded) to fix m_ref,
    // then its partner half published for step 0
    // tile 0 landed; tiles 1, 2 (and the fourth tile's page-table entries) may be in flight
    if (attempt == 0) {
      // tile 0 and the queries landed; tile 1 (paged: and the fourth tile's
      // page-table entries) may be in flight
      if (kPaged)
        __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10)
      else
        __builtin_amdgcn_s_waitcnt(0x0F79);  // vmcnt(9)
      __syncthreads();
      // rows 32 hh .. 32 hh + 31 of the block, this wave's dim half
      if (hh == 0) {
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) qreg[ks] = lds_b128(r3 + k_frag_off<kDh>(kb, ks));
      } else {
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) qreg[ks] = lds_b128(r2 + k_frag_off<kDh>(kb, ks));
      }
      __syncthreads();  // every wave holds its queries: slots 2 and 3 are free
    }
    // tile 2 (in the redo: again, the same bytes; outside the branch so that
    // the compiler's LDS-DMA tracking keeps the first steps' waits relaxed)
    if constexpr (kPaged)
      issue_paged(r2, checked_idx(2, idx2));
    else
      issue_tile(r2, lat_rs, rope_rs, tile_rel(2), wave, lane, rope_voff);
    // (the redo's first tiles were loaded and drained at the end of the
    // first attempt: no load crosses the back edge, so that at this join the
    // compiler's LDS-DMA tracking still tells the ring slots apart and keeps
    // the waits of the first steps relaxed)
    const f32x16_t s0 = tile_scores<kDh>(r0, qreg, kb);
    float own[8];  // this wave's elements of the next tile's partial scores
#pragma unroll
    for (int k = 0; k < 8; ++k) own[k] = s0[kOwn + k];
    if (attempt == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *(LDS_AS f32x4_t*)(r3 + wave * 4096 + c * 1024 + lane * 16) =
            (f32x4_t){s0[4 * c], s0[4 * c + 1], s0[4 * c + 2], s0[4 * c + 3]};
      lds_barrier();  // (tile 2 may be in flight: no fence)
      const uint32_t vis0 = tile_visibility(c0, c1, prefix, anc);
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4_t p4 = *(const LDS_AS f32x4_t*)(r3 + partner * 4096 + c * 1024 + lane * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (key_visible_bit(vis0, 4 * c + e)) mx = fmax3(mx, s0[4 * c + e] + p4[e]);
      }
      have_ref = vis0 != 0;
      m_ref = have_ref ? partner_max(mx) * sl2 + kRefShift : -INFINITY;
    }
    *(LDS_AS f32x4_t*)(xs_mine) = (f32x4_t){s0[kSend], s0[kSend + 1], s0[kSend + 2], s0[kSend + 3]};
    *(LDS_AS f32x4_t*)(xs_mine + 1024) =
        (f32x4_t){s0[kSend + 4], s0[kSend + 5], s0[kSend + 6], s0[kSend + 7]};

    // One step: softmax (own keys) and values (all keys) of tile i, scores
    // of tile i+1 (computed even past the last tile, on whatever that ring
    // slot holds, and unused then), loads of tile i+3 into the free slot.
    // The body is an explicit software pipeline over MFMA slots: each LDS
    // operand is read kAhead slots before its use, and the softmax is cut
    // into slices of about one MFMA's issue budget placed behind the score
    // MFMAs (a wave issues one instruction per 4 cycles, eight per 32-cycle
    // MFMA). sched_barrier fences keep the slots in this order. Between the
    // score and the value phases the waves meet at a barrier, after which
    // each reads its partner's weights. kMasked selects the per-key
    // visibility test (and the first-visible-tile path).
    // Tile i+1 landed (tile i+2 may still be in flight) and the partner
    // scores of tile i are published once every wave passes the barrier;
    // ring slot (i+3)%4 is free from then on.
    auto advance = [&]() {
      // only tile i+2's loads (and, paged, the page-table load before them) may be outstanding
      if (kPaged)
        __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10)
      else
        __builtin_amdgcn_s_waitcnt(0x0F79);  // vmcnt(9)
      lds_barrier();
    };
    // The first kAhead K-operand reads of the next step, issued before the
    // last value MFMAs of the current one so that their LDS latency hides
    // behind those MFMAs instead of stalling the next step's first score MFMA.
    constexpr int kAhead = 8;
    bf16x8_t kpre[kAhead];
    auto prefetch_k = [&](LDS_AS char* nbuf) {
#pragma unroll
      for (int ks = 0; ks < kAhead; ++ks) {
        kpre[ks] = lds_b128(nbuf + k_frag_off<kDh>(kb, ks));
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // kbuf: tile i+1 (scores), vbuf: tile i (values), dma_buf: the slot that
    // takes tile i+3, nbuf: tile i+2 (the next step's scores)
    auto step = [&](auto masked_tag, LDS_AS char* kbuf, LDS_AS char* vbuf, LDS_AS char* dma_buf,
                    LDS_AS char* nbuf, int i, uint32_t vis) {
      constexpr bool kMasked = decltype(masked_tag)::value;
      const int dma_rel = tile_rel(i + 3);
      auto kread = [&](int ks) { return lds_b128(kbuf + k_frag_off<kDh>(kb, ks)); };
      // fragment order: the wave's own key step first (its weights are ready
      // first), then the partner's
      auto frag = [&](int nn) { return nn < 8 ? 8 * kDh + nn : 8 * (1 - kDh) + (nn - 8); };
      auto vread = [&](int j) {  // dim block j&7 of this wave's 256 dims, key step j>>3
        const int dbg = 8 * kDh + (j & 7);
        const int off = 256 * (dbg >> 2) + 16 * 1024 * (j >> 3);
        const int m0 = (dbg & 1) + 2 * ((dbg >> 1) & 1);  // keys +0..3 (v = 0)
        const int m1 = m0 ^ 2;                             // keys +8..11 (v = 1)
        const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)(vbuf + vb[m0] + off));
        const bf16x4_t v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)(vbuf + vb[m1] + off + 8 * 1024));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };

      // the partner's partial scores of this wave's keys of tile i
      const f32x4_t pa = *(const LDS_AS f32x4_t*)(xs_part);
      const f32x4_t pb = *(const LDS_AS f32x4_t*)(xs_part + 1024);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t kf[18], vf[16];
#pragma unroll
      for (int ks = 0; ks < kAhead; ++ks) kf[ks] = kpre[ks];  // read during the previous step

      f32x16_t sc = {};
      float sv[8], pw[8];
      float smax = 0.f, mref = 0.f;
      u32x4_t ph[2], pl[2];  // bf16 pairs of the P^T operand (hi and lo parts), per key step
      auto weight = [&](int k) { pw[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[k], sl2, -mref)); };
      // own weights k, k+1 -> operand words: hi = the weight rounded to bf16,
      // lo = the exact remainder rounded to bf16, so that hi + lo carries
      // about 17 significant bits.
      auto split_pair = [&](int k) {
        l_run += pw[k] + pw[k + 1];
        const bf16x2_t h2 = {(__bf16)pw[k], (__bf16)pw[k + 1]};
        const uint32_t hi = __builtin_bit_cast(uint32_t, h2);
        uint32_t lo = 0;
        if (kHiLo) {
          const bf16x2_t l2 = {(__bf16)(pw[k] - __uint_as_float(hi << 16)),
                               (__bf16)(pw[k + 1] - __uint_as_float(hi & 0xffff0000u))};
          lo = __builtin_bit_cast(uint32_t, l2);
        }
        ph[kDh][k >> 1] = hi;
        pl[kDh][k >> 1] = lo;
      };

      // scores of tile i+1; softmax of this wave's keys of tile i behind them
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qreg[ks], sc, 0, 0, 0);
        if (ks + kAhead < 18)
          kf[ks + kAhead] = kread(ks + kAhead);
        else
          vf[frag(ks + kAhead - 18)] = vread(frag(ks + kAhead - 18));
        if (ks == 0) {
#pragma unroll
          for (int k = 0; k < 4; ++k) sv[k] = own[k] + pa[k];
        } else if (ks == 1) {
#pragma unroll
          for (int k = 0; k < 4; ++k) sv[4 + k] = own[4 + k] + pb[k];
        } else if (ks == 2) {
          if (kMasked) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (!key_visible_bit(vis, kOwn + k)) sv[k] = -INFINITY;
          }
          smax = sv[0];
#pragma unroll
          for (int k = 1; k < 8; ++k) smax = fmax3(smax, sv[k]);
        } else if (ks == 3) {
          const float mt = partner_max(smax) * sl2;  // max over this wave's 16 keys
          m_seen = fmax3(m_seen, mt);
          if (kMasked && ref_xchg) {
            // a row's first tile with a visible key: both halves' maxes fix its m_ref
            __syncthreads();  // every wave has consumed its partner's scores
            *(LDS_AS float*)(xs + wave * 2048 + lane * 4) = mt;
            __syncthreads();
            const bool adopt = !have_ref && vis != 0;
            m_ref = adopt ? fmax3(mt, *(const LDS_AS float*)(xs + partner * 2048 + lane * 4)) + kRefShift : m_ref;
            have_ref = have_ref || adopt;
          }
          ovf |= mt > m_ref + kRefHeadroom;
          mref = m_ref == -INFINITY ? 0.f : m_ref;
        } else if (ks >= 4 && ks < 8) {
          weight(2 * (ks - 4));
          weight(2 * (ks - 4) + 1);
        } else if (ks >= 8 && ks < 12) {
          split_pair(2 * (ks - 8));
        } else if (ks == 12) {
          *(LDS_AS u32x4_t*)(xp_mine) = ph[kDh];
          *(LDS_AS u32x4_t*)(xp_mine + 1024) = pl[kDh];
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // every wave's weights are published; every wave has read its partner's
      // partial scores of tile i, so the exchange area can take tile i+1's
      lds_barrier();
      ph[1 - kDh] = *(const LDS_AS u32x4_t*)(xp_part);
      pl[1 - kDh] = *(const LDS_AS u32x4_t*)(xp_part + 1024);
      *(LDS_AS f32x4_t*)(xs_mine) = (f32x4_t){sc[kSend], sc[kSend + 1], sc[kSend + 2], sc[kSend + 3]};
      *(LDS_AS f32x4_t*)(xs_mine + 1024) =
          (f32x4_t){sc[kSend + 4], sc[kSend + 5], sc[kSend + 6], sc[kSend + 7]};
      __builtin_amdgcn_sched_barrier(0);

      // paged KV: this step's loads use the page-table entries read one step
      // ago; the next tile's entries are requested before them
      int idx_dma = 0, rope_dma = 0, idx_next = 0;
      if constexpr (kPaged) {
        idx_dma = checked_idx(i + 3, idx_cur);
        rope_dma = rope_rows(idx_dma);
        idx_next = load_idx(i + 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      // values of tile i; tile loads in the first slots (each slot holds two
      // MFMAs, so it has issue room to spare). Before the last kTail value
      // slots the waves meet for the next step (tile i+2 landed, the partner
      // scores of tile i+1 published) and the next step's first K operands
      // are requested; those value MFMAs then cover the LDS latency.
      constexpr int kTail = 2;
#pragma unroll
      for (int nn = 0; nn < 16; ++nn) {
        if (nn == 16 - kTail) {
          advance();
          prefetch_k(nbuf);
        }
        const int j = frag(nn);
        acc[j & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j], __builtin_bit_cast(bf16x8_t, ph[j >> 3]),
                                                             acc[j & 7], 0, 0, 0);
        if (kHiLo)
          acc[j & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j], __builtin_bit_cast(bf16x8_t, pl[j >> 3]),
                                                               acc[j & 7], 0, 0, 0);
        if (nn + kAhead < 16) vf[frag(nn + kAhead)] = vread(frag(nn + kAhead));
        if (kPaged) {
          if (nn < 9) issue_tile_part_paged(dma_buf, lat_rs, rope_rs, idx_dma, rope_dma, wave, lane, rope_loff, nn);
        } else {
          if (nn < 9) issue_tile_part(dma_buf, lat_rs, rope_rs, dma_rel, wave, lane, rope_voff, nn);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) own[k] = sc[kOwn + k];
      if constexpr (kPaged) idx_cur = idx_next;
    };

    // Tiles wholly inside the prefix and the chunk need no mask. Their loop
    // is unrolled by the ring period so that every step's slots are
    // compile-time objects; the remaining tiles take the masked step with the
    // slots chosen at run time (for those the compiler cannot rule out that
    // the tile being loaded is read, so it waits for the load). Separate
    // loops keep a single register assignment per loop body.
    const int64_t full_end = prefix < c1 ? prefix : c1;
    const int n_full = full_end > c0 ? (int)((full_end - c0) / kTile) : 0;
    // each step ends by meeting the other waves for the next one and reading
    // its first K operands; the first step's are read here
    advance();
    prefetch_k(r1);
    int i = 0;
    for (; i + 4 <= n_full; i += 4) {
      step(std::false_type{}, r1, r0, r3, r2, i, 0u);
      step(std::false_type{}, r2, r1, r0, r3, i + 1, 0u);
      step(std::false_type{}, r3, r2, r1, r0, i + 2, 0u);
      step(std::false_type{}, r0, r3, r2, r1, i + 3, 0u);
    }
    // up to three more whole tiles: i is a multiple of 4 here, so their ring
    // slots are still compile-time objects
    if (i < n_full) {
      step(std::false_type{}, r1, r0, r3, r2, i, 0u);
      ++i;
      if (i < n_full) {
        step(std::false_type{}, r2, r1, r0, r3, i, 0u);
        ++i;
        if (i < n_full) {
          step(std::false_type{}, r3, r2, r1, r0, i, 0u);
          ++i;
        }
      }
    }
    for (; i < ntiles; ++i) {
      const uint32_t vis = tile_visibility(c0 + (int64_t)i * kTile, c1, prefix, anc);
      step(std::true_type{}, ring((i + 1) & 3), ring(i & 3), ring((i + 3) & 3), ring((i + 2) & 3), i, vis);
    }
    // Accumulator overflow: weights reach 2^96 before a redo, so values of
    // 2^32 / (keys in the chunk) and more can push a sum past fp32. The
    // largest |accumulator| of the lane (also the int16 quantisation's row
    // maximum below) catches it, and the chunk is then redone with its own
    // maximum as the reference (weights at most 1). Below 2^31 no single
    // product overflows, so a sum that overflowed holds an infinity, which
    // this maximum sees.
    {
      float mx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int e = 0; e < 16; e += 2)
          mx[(e >> 1) & 3] = max3_abs(mx[(e >> 1) & 3], acc[db][e], acc[db][e + 1]);
      acc_amax = fmax3(fmax3(mx[0], mx[1]), fmax3(mx[2], mx[3]));
      ovf |= !(acc_amax <= 3.402823466e38f);
    }
    // workgroup-wide OR of the overflow flags, through the exchange area
    // (every wave is past its last read of it once all pass the barrier)
    __syncthreads();
    const int wave_ovf = __builtin_amdgcn_ballot_w64(ovf != 0) != 0;  // OR over this wave's heads
    if (lane == 0) *(LDS_AS int*)(xs + wave * 2048) = wave_ovf;
    __syncthreads();
    const int any_ovf = *(const LDS_AS int*)(xs) | *(const LDS_AS int*)(xs + 2048) |
                        *(const LDS_AS int*)(xs + 4096) | *(const LDS_AS int*)(xs + 6144);
    __syncthreads();
    if (!any_ovf) break;
    // redo with m_ref = the chunk's max over both waves' keys
    *(LDS_AS float*)(xs + wave * 2048 + lane * 4) = m_seen;
    __syncthreads();
    m_ref = fmax3(m_seen, *(const LDS_AS float*)(xs + partner * 2048 + lane * 4));
    have_ref = true;
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    restart_tiles();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tiles 0..2 (paged: and the fourth tile's entries) landed
    __syncthreads();
  }

  // denominator: this lane pair's own keys, plus the partner wave's keys
  // (no tile load is in flight and every wave is past its last LDS read)
  float l_tot = partner_sum(l_run);
  *(LDS_AS float*)(xs + wave * 2048 + lane * 4) = l_tot;
  __syncthreads();
  l_tot += *(const LDS_AS float*)(xs + partner * 2048 + lane * 4);

  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_val = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  const bool final_write = nsplit_b == 1;
  const bool compact = kCompact && !final_write;
  const int64_t out_row0 = (int64_t)b * rows_seq + rbk * kRows;  // first output row of the block
  const int nvalid = rows_seq - rbk * kRows < kRows ? rows_seq - rbk * kRows : kRows;
  const int64_t prow = (((int64_t)b * a.nsplit + s) * a.nrb + rbk) * kRows;  // first partial row
  // fp32 partials keep the padded row block (all 64 rows); int16 partials and
  // the final output take the block's rows below q * heads only.
  if (compact) {
    // Compact partials: row h of the normalised partial is stored as 512
    // int16 values q with one fp32 scale, value = q * scale, where scale =
    // (largest |value| of the row) / 32767; rounding to nearest keeps every
    // value within scale / 2, i.e. 2^-16 of the row's largest.
    // The quantisation runs in the accumulator layout: lane (head, half)
    // holds dims 256 kDh + 32 db + 8 g + 4 half + e of its row in acc[db][4 g
    // + e], so the row max is an in-lane max, one lane-pair swap and one
    // exchange with the partner wave (the other 256 dims), and adjacent dims
    // sit in adjacent elements, which v_cvt_pknorm_i16_f32 packs pairwise.
    // One lane-pair swap per two 8-byte pieces gives each lane 16 bytes (8
    // dims) of its row, the two lanes of a row holding the two halves of one
    // 16-dim pair. The block's values lie pair-major in the workspace
    // ([32 pairs][64 rows][16 dims], 32 B per row and pair), so every store
    // leaves straight from registers as 1 KB (32 rows x 32 B of one pair).
    float m = partner_max(acc_amax);
    *(LDS_AS float*)(xs + wave * 2048 + 1024 + lane * 4) = m;  // clear of the l_tot words read above
    __syncthreads();
    m = fmax3(m, *(const LDS_AS float*)(xs + partner * 2048 + 1024 + lane * 4));  // largest |acc| of the row
    // acc / m lies in [-1, 1]; v_cvt_pknorm_i16_f32 scales by 32767, rounds
    // to nearest and packs two values
    const float g = m > 0.f ? __builtin_amdgcn_rcpf(m) : 0.f;
    auto q2 = [&](float x, float y) {
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(x * g, y * g));
    };
    // The partial rows leave with device-scope stores (sc1: written through
    // the XCD's L2). A block merged in this kernel needs that (another
    // workgroup, maybe on another XCD, reads the rows at once); for the
    // combine kernel it is measured 1 us faster per call at q 9, H 64,
    // prefix 16384 than write-back stores, whose dirty lines the release at
    // the kernel's end must write back before the combine can start.
    // Rows past q * heads (the padding of the last block) are not stored: no
    // merge reads them for an output, and each row merges on its own.
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(a.part_q + prow * kDl, kRows * kDl * 2);
    const bool store_row = head < nvalid;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const uint32_t a0 = q2(acc[db][8 * gp], acc[db][8 * gp + 1]);
        const uint32_t a1 = q2(acc[db][8 * gp + 2], acc[db][8 * gp + 3]);
        const uint32_t b0 = q2(acc[db][8 * gp + 4], acc[db][8 * gp + 5]);
        const uint32_t b1 = q2(acc[db][8 * gp + 6], acc[db][8 * gp + 7]);
        const auto x = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto y = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        const int pair = 16 * kDh + 2 * db + gp;  // dims [16 pair, 16 pair + 16)
        if (store_row)
          __builtin_amdgcn_raw_buffer_store_b128((u32x4_t){x[0], y[0], x[1], y[1]}, prs,
                                                 compact_byte_off(pair, head) + 16 * half, 0, kCoherent);
      }
    }
    if (kDh == 0 && half == 0)
      __hip_atomic_store(a.part_scale + prow + head, m * inv * (1.f / 32767.f), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  } else {
    // Stage the accumulators through LDS so that each global store writes
    // two 512-byte row pieces instead of 32-byte pieces of 32 rows. Ring
    // slot o takes dims [128 o, 128 o + 128) of all 64 rows (the slot of a
    // write is then a compile-time choice); row h's 32 16-byte chunks sit at
    // h * 512 + 16 * (c ^ (h & 15)), conflict-free for the row-per-lane
    // writes and the chunk-per-lane reads. The reads apply 1 / l, kept per
    // row in the weight-exchange area.
    if (kDh == 0 && half == 0) *(LDS_AS float*)(xp + head * 4) = inv;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      LDS_AS char* slot = ring(2 * kDh + (db >> 2));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 8 * (db & 3) + 2 * g + half;
        *(LDS_AS f32x4_t*)(slot + head * 512 + 16 * (c ^ (head & 15))) =
            (f32x4_t){acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
      }
    }
    __syncthreads();
    float* obase = final_write ? a.out + out_row0 * kDl : a.part_o + prow * kDl;
    const int nstore = final_write ? nvalid : kRows;
    // this wave stores ring slot `wave`: dims [128 wave, 128 wave + 128)
    LDS_AS char* slot = ring(wave);
    const int c = lane & 31;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int h = 2 * k + half;
      const f32x4_t v = *(const LDS_AS f32x4_t*)(slot + h * 512 + 16 * (c ^ (h & 15)));
      const float sc_h = *(const LDS_AS float*)(xp + h * 4);
      if (h < nstore) *(f32x4_t*)(obase + (int64_t)h * kDl + 128 * wave + 4 * c) = v * sc_h;
    }
  }
  if (kDh == 0 && half == 0) {
    if (final_write) {
      if (head < nvalid) a.lse[out_row0 + head] = lse_val;
    } else if (kCompact) {
      __hip_atomic_store(a.part_lse + prow + head, lse_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      a.part_lse[prow + head] = lse_val;
    }
  }
}

template <bool kHiLo, bool kCompact, bool kPaged, bool kFused>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void split_mfma_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char ring0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char ring1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char ring2[kTileBytes];
  __shared__ __attribute__((aligned(16))) char ring3[kTileBytes];
  __shared__ __attribute__((aligned(16))) char xs_raw[kXchgBytes];
  __shared__ __attribute__((aligned(16))) char xp_raw[kXchgBytes];
  LDS_AS char* r0 = (LDS_AS char*)ring0;
  LDS_AS char* r1 = (LDS_AS char*)ring1;
  LDS_AS char* r2 = (LDS_AS char*)ring2;
  LDS_AS char* r3 = (LDS_AS char*)ring3;
  LDS_AS char* xs = (LDS_AS char*)xs_raw;
  LDS_AS char* xp = (LDS_AS char*)xp_raw;
  // Fetch the kernel arguments the prologue needs in one round of scalar
  // loads (fetched lazily, each group would wait on its own round trip).
  asm volatile("" ::"s"(a.qn), "s"(a.qr), "s"(a.lat), "s"(a.rope), "s"(a.parent), "s"(a.offs),
               "s"(a.single_n), "s"(a.total_kv), "s"(a.max_kv), "s"(a.chunk), "s"(a.scale_log2), "s"(a.q),
               "s"(a.heads), "s"(a.nrb), "s"(a.nsplit), "s"(a.nwork), "s"(a.per_xcd), "s"(a.batch),
               "s"(a.list_run));
  int b, s, t;  // t: the row block
  int64_t row0, n;
  bool ok;
  if (a.list_run > 0) {
    if (!decode_list(a, b, s, t, row0, n, ok)) return;
  } else {
    if (!decode_work(a, b, s, t)) return;
    ok = seq_bounds(a, b, row0, n);
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  if (!ok) {
    if (s == 0) write_nan_rows(a, b, t, tid, kThreads);
    return;
  }
  row0 = uniform64(row0);
  n = uniform64(n);
  if ((int64_t)s * a.chunk >= n) return;  // this sequence needs fewer splits
  const int hh = wave >> 1;
  if ((wave & 1) == 0)
    split_body<0, kHiLo, kCompact, kPaged, kFused>(a, r0, r1, r2, r3, xs, xp, b, s, t, wave, hh, lane, row0, n);
  else
    split_body<1, kHiLo, kCompact, kPaged, kFused>(a, r0, r1, r2, r3, xs, xp, b, s, t, wave, hh, lane, row0, n);
  if constexpr (kFused) {
    static_assert(kCompact, "the merge in the split kernel reads int16 partials");
    switch ((int)((n + a.chunk - 1) / a.chunk)) {  // this sequence's splits
      case 2: merge_block<2>(a, xs, b, t, wave, lane); break;
      case 3: merge_block<3>(a, xs, b, t, wave, lane); break;
      case 4: merge_block<4>(a, xs, b, t, wave, lane); break;
      default: break;  // one split: out and lse are written
    }
  }
}

// ---------------------------------------------------------------------------
// split kernel: plain fp32 VALU (second implementation, for cross-checks)
// one wave per (token, head, split); keys processed one at a time
// ---------------------------------------------------------------------------
__device__ inline float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__global__ __launch_bounds__(kThreads) void split_valu_kernel(Args a) {
  const int work = blockIdx.x >> 4;  // 16 workgroups x 4 waves = the 64 rows of a row block
  const int head = ((blockIdx.x & 15) << 2) + (threadIdx.x >> 6);  // row in the block
  const int lane = threadIdx.x & 63;
  if (work >= a.nwork) return;
  const int rbk = work % a.nrb;
  const int s = (work / a.nrb) % a.nsplit;
  const int b = work / (a.nrb * a.nsplit);
  int64_t row0, n;
  if (!seq_bounds(a, b, row0, n)) {
    if (s == 0 && (blockIdx.x & 15) == 0) write_nan_rows(a, b, rbk, threadIdx.x, kThreads);
    return;
  }
  const int rows_seq = a.q * a.heads;
  const int r = rbk * kRows + head;  // (token, head) row of the sequence
  if (r >= rows_seq) return;
  const int t = r / a.heads;
  const int64_t prefix = n - a.q;
  const int64_t c0 = (int64_t)s * a.chunk;
  if (c0 >= n) return;
  const int64_t c1 = c0 + a.chunk < n ? c0 + a.chunk : n;
  const int nsplit_b = (int)((n + a.chunk - 1) / a.chunk);
  const uint64_t anc = ancestor_mask(a.parent + (int64_t)b * a.q, a.q, t);
  const int64_t qrow = (int64_t)b * rows_seq + r;

  // lane owns query dims [8 lane, 8 lane + 8) of the latent part and dim `lane` of the rope part
  float qv[9];
  for (int d = 0; d < 8; ++d) qv[d] = bf16_to_f32(a.qn[qrow * kDl + 8 * lane + d]);
  qv[8] = bf16_to_f32(a.qr[qrow * kDr + lane]);
  float m = -INFINITY, l = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t j = c0; j < c1; ++j) {
    if (!key_visible(j, c1, prefix, anc)) continue;
    // contiguous KV: row row0 + j; paged KV: the pool row the page table
    // gives, a row outside the pool reading as zeros (as in the MFMA kernel)
    int64_t krow = row0 + j;
    bool zero = false;
    if (a.idx) {
      const int pr = a.idx[row0 + j];
      zero = pr < 0 || pr >= a.pool_rows;
      krow = zero ? 0 : pr;
    }
    const uint16_t* kl = a.lat + krow * kDl + 8 * lane;
    float v[8];
    float part = 0.f;
    for (int d = 0; d < 8; ++d) {
      v[d] = zero ? 0.f : bf16_to_f32(kl[d]);
      part += qv[d] * v[d];
    }
    part += qv[8] * (zero ? 0.f : bf16_to_f32(a.rope[krow * kDr + lane]));
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    const float sj = part * a.scale_log2;
    const float m_new = fmax3(m, sj);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    const float p = __builtin_amdgcn_exp2f(sj - m_new);
    l = l * alpha + p;
    for (int d = 0; d < 8; ++d) acc[d] = acc[d] * alpha + p * v[d];
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse_val = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  const bool final_write = nsplit_b == 1;
  const int64_t prow = (((int64_t)b * a.nsplit + s) * a.nrb + rbk) * kRows + head;  // padded partial row
  float* orow = final_write ? a.out + qrow * kDl : a.part_o + prow * kDl;
  for (int d = 0; d < 8; ++d) orow[8 * lane + d] = acc[d] * inv;
  if (lane == 0) {
    if (final_write)
      a.lse[qrow] = lse_val;
    else
      a.part_lse[prow] = lse_val;
  }
}

// Every argument a combine kernel uses, in one round of scalar loads
// (fetched lazily they took three dependent rounds, each a memory round trip
// at kernel start).
__device__ inline void fetch_combine_args(const Args& a, int64_t rows) {
  asm volatile("" ::"s"(rows), "s"(a.q), "s"(a.heads), "s"(a.nrb), "s"(a.nsplit), "s"(a.chunk), "s"(a.offs),
               "s"(a.single_n), "s"(a.total_kv), "s"(a.max_kv), "s"(a.part_q), "s"(a.part_o), "s"(a.part_lse),
               "s"(a.part_scale), "s"(a.out), "s"(a.lse), "s"(a.fixed_ns));
}

// ---------------------------------------------------------------------------
// combine: log-sum-exp merge of the split partials, 128 threads per row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void combine_kernel(Args a, int64_t rows) {
  fetch_combine_args(a, rows);
  const int64_t row = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  if (row >= rows) return;
  const int d4 = threadIdx.x & 127;
  const int64_t rows_b = (int64_t)a.q * a.heads;      // output rows per sequence
  const int64_t rows_pad = (int64_t)a.nrb * kRows;     // partial rows per (sequence, split)
  const int b = (int)(row / rows_b);
  const int64_t rb = row - (int64_t)b * rows_b;
  int ns = a.fixed_ns;
  if (ns <= 0) {
    int64_t row0, n;
    if (!seq_bounds(a, b, row0, n)) {
      const float nan = __builtin_nanf("");
      *(f32x4_t*)(a.out + row * kDl + 4 * d4) = (f32x4_t){nan, nan, nan, nan};
      if (d4 == 0) a.lse[row] = nan;
      return;
    }
    ns = (int)((n + a.chunk - 1) / a.chunk);
    if (ns <= 1) return;  // the split kernel wrote this row directly
  }
  const float* pl = a.part_lse + (int64_t)b * a.nsplit * rows_pad + rb;
  const float* po = a.part_o + ((int64_t)b * a.nsplit * rows_pad + rb) * kDl + 4 * d4;
  // Batches of up to 32 splits: every lse and partial load of a batch is
  // issued before any is used (one memory round trip per batch); batches are
  // merged with a running max. Entries past the last split reload the last
  // one and get weight 0 (partials are finite), so the loads need no branches;
  // splits are still added in order.
  constexpr int kBatch = 32;
  float M = -INFINITY;
  f32x4_t accv = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kBatch) {
    f32x4_t o[kBatch];
    float lz[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int sk = s0 + k < ns ? s0 + k : ns - 1;
      lz[k] = pl[(int64_t)sk * rows_pad];
      o[k] = __builtin_nontemporal_load((const f32x4_t*)(po + (int64_t)sk * rows_pad * kDl));
    }
    float mb = -INFINITY;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mb = fmax3(mb, lz[k]);  // reloaded entries repeat a real one
    if (mb == -INFINITY) continue;  // every split of this batch is empty
    const float m_new = fmax3(M, mb);
    const float r = __builtin_amdgcn_exp2f((M - m_new) * kLog2e);  // 0 while M = -inf
    accv *= r;
    wsum *= r;
    M = m_new;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = s0 + k < ns ? __builtin_amdgcn_exp2f((lz[k] - M) * kLog2e) : 0.f;
      wsum += w;
      accv += w * o[k];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *(f32x4_t*)(a.out + row * kDl + 4 * d4) = accv * inv;
  if (d4 == 0) a.lse[row] = wsum > 0.f ? M + __builtin_amdgcn_logf(wsum) * kLn2 : -INFINITY;
}

// Combine of compact (int16 + scale) partials. A work unit is (sequence b,
// row block t, 16-dim pair p, row half rh): 32 rows x 16 dims, whose 32-byte
// pieces lie one after another in every split's pair-major block, so each
// partial load of a wave reads 1 KB contiguous. Lane (i, half) takes row
// 32 rh + i of the block and dims 16 p + 8 half .. + 8, fetches its row's
// lse and scale of every split itself, and merges with a running max.
struct CombineUnit {
  int b, t, p, h, half;
  int64_t row;    // output row (sequence b's row t * 64 + h)
  bool valid;     // the row exists (rows past q * heads pad the last block)
};

__device__ inline CombineUnit combine_unit(const Args& a, int64_t unit, int lane) {
  CombineUnit u;
  const int rh = (int)(unit & 1);
  u.p = (int)((unit >> 1) & 31);
  const int64_t bt = unit >> 6;
  u.b = (int)(bt / a.nrb);
  u.t = (int)(bt - (int64_t)u.b * a.nrb);
  u.h = 32 * rh + (lane & 31);
  u.half = lane >> 5;
  const int64_t rows_b = (int64_t)a.q * a.heads;
  const int64_t r = (int64_t)u.t * kRows + u.h;
  u.valid = r < rows_b;
  u.row = (int64_t)u.b * rows_b + r;
  return u;
}

// NaN rows of a sequence with inconsistent offsets (this lane's 8 dims).
__device__ inline void combine_nan(const Args& a, const CombineUnit& u) {
  if (!u.valid) return;
  const float nan = __builtin_nanf("");
  float* o = a.out + u.row * kDl + 16 * u.p + 8 * u.half;
  *(f32x4_t*)o = (f32x4_t){nan, nan, nan, nan};
  *(f32x4_t*)(o + 4) = (f32x4_t){nan, nan, nan, nan};
  if (u.p == 0 && u.half == 0) a.lse[u.row] = nan;
}

// Merges splits [s_lo, s_hi) of the unit's lane into (M, wsum, acc), kBatch
// splits per memory round trip (every load of a batch issued first; entries
// past s_hi reload the last split and get weight 0); batches meet through a
// running max.
template <int kBatch>
__device__ inline void combine_splits(const Args& a, const CombineUnit& u, int s_lo, int s_hi, float& M,
                                      float& wsum, float (&acc)[8]) {
  const int64_t sstride = (int64_t)a.nrb * kRows;                         // partial rows between splits
  const int64_t prow0 = ((int64_t)u.b * a.nsplit * a.nrb + u.t) * kRows;  // split 0's block
  const int16_t* pq = a.part_q + prow0 * kDl + compact_byte_off(u.p, u.h) / 2 + 8 * u.half;
  // the row's lse (lanes of half 0) or scale (half 1): one load per split,
  // and a swap of the two lane halves gives every lane both
  const float* pv = (u.half ? a.part_scale : a.part_lse) + prow0 + u.h;
  for (int s0 = s_lo; s0 < s_hi; s0 += kBatch) {
    u32x4_t qv[kBatch];
    float vv[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int sk = s0 + k < s_hi ? s0 + k : s_hi - 1;
      qv[k] = __builtin_nontemporal_load((const u32x4_t*)(pq + (int64_t)sk * sstride * kDl));
      vv[k] = pv[(int64_t)sk * sstride];
    }
    float lz[kBatch], sc[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(vv[k]), __float_as_uint(vv[k]), false, false);
      lz[k] = __uint_as_float(x[0]);
      sc[k] = __uint_as_float(x[1]);
    }
    float mb = -INFINITY;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mb = fmax3(mb, lz[k]);  // reloaded entries repeat a real one
    if (mb == -INFINITY) continue;  // every split of this batch is empty for this row
    const float m_new = fmax3(M, mb);
    const float r = __builtin_amdgcn_exp2f((M - m_new) * kLog2e);  // 0 while M = -inf
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= r;
    wsum *= r;
    M = m_new;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = s0 + k < s_hi ? __builtin_amdgcn_exp2f((lz[k] - M) * kLog2e) : 0.f;
      wsum += w;
      const float f = w * sc[k];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int32_t v = (int32_t)qv[k][e];
        acc[2 * e] += f * (float)((v << 16) >> 16);
        acc[2 * e + 1] += f * (float)(v >> 16);
      }
    }
  }
}

__device__ inline void combine_store(const Args& a, const CombineUnit& u, float M, float wsum,
                                     const float (&acc)[8]) {
  if (!u.valid) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float* o = a.out + u.row * kDl + 16 * u.p + 8 * u.half;
  // streaming stores: the rows are not read again by this GPU before the call ends
  __builtin_nontemporal_store((f32x4_t){acc[0], acc[1], acc[2], acc[3]} * inv, (f32x4_t*)o);
  __builtin_nontemporal_store((f32x4_t){acc[4], acc[5], acc[6], acc[7]} * inv, (f32x4_t*)(o + 4));
  if (u.p == 0 && u.half == 0) a.lse[u.row] = wsum > 0.f ? M + __builtin_amdgcn_logf(wsum) * kLn2 : -INFINITY;
}

// Up to 32 splits: one wave per unit, all of a row's loads in one round
// trip (kBatch loads per lane, the plan's split count rounded up to a
// multiple of 4).
template <int kBatch>
__global__ __launch_bounds__(64) void combine_compact_kernel(Args a, int64_t units) {
  fetch_combine_args(a, units);
  const int64_t unit = blockIdx.x;
  if (unit >= units) return;
  const CombineUnit u = combine_unit(a, unit, threadIdx.x & 63);
  int64_t row0, n;
  if (!seq_bounds(a, u.b, row0, n)) {
    combine_nan(a, u);
    return;
  }
  const int ns = (int)((n + a.chunk - 1) / a.chunk);
  if (ns <= 1) return;  // the split kernel wrote this row directly
  float M = -INFINITY, wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  combine_splits<kBatch>(a, u, 0, ns, M, wsum, acc);
  combine_store(a, u, M, wsum, acc);
}

// More than 32 splits: four waves per unit; wave w merges splits
// [w ns / 4, (w + 1) ns / 4) in batches of kBatch (its share of the plan's
// splits rounded up to a multiple of 4, at most 32), and the four partial
// merges meet in LDS.
template <int kBatch>
__global__ __launch_bounds__(kThreads) void combine_compact_wide_kernel(Args a, int64_t units) {
  fetch_combine_args(a, units);
  __shared__ float x_acc[4][8][64];
  __shared__ float x_m[4][64], x_w[4][64];
  const int64_t unit = blockIdx.x;
  if (unit >= units) return;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const CombineUnit u = combine_unit(a, unit, lane);
  int64_t row0, n;
  if (!seq_bounds(a, u.b, row0, n)) {
    if (wave == 0) combine_nan(a, u);
    return;
  }
  const int ns = (int)((n + a.chunk - 1) / a.chunk);
  if (ns <= 1) return;  // the split kernel wrote this row directly
  float M = -INFINITY, wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int s_lo = wave * ns / 4, s_hi = (wave + 1) * ns / 4;
  if (s_lo < s_hi) combine_splits<kBatch>(a, u, s_lo, s_hi, M, wsum, acc);
#pragma unroll
  for (int e = 0; e < 8; ++e) x_acc[wave][e][lane] = acc[e];
  x_m[wave][lane] = M;
  x_w[wave][lane] = wsum;
  __syncthreads();
  if (wave != 0) return;
  float mm = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) mm = fmax3(mm, x_m[w][lane]);
  float tot = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (mm != -INFINITY) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float r = __builtin_amdgcn_exp2f((x_m[w][lane] - mm) * kLog2e);  // 0 for a wave with nothing
      tot += r * x_w[w][lane];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += r * x_acc[w][e][lane];
    }
  }
  combine_store(a, u, mm, tot, o);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Static device scratch for callers that cannot allocate (mla_verify_noalloc):
// the split partials of one call live here instead of in a caller workspace.
// Each device holds its own copy for the life of the process. The array's
// name is a host-side stand-in in host code; kernels get the device address
// that hipGetSymbolAddress returns, looked up once per device.
static __device__ __attribute__((aligned(256))) char scratch[MLAV_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device (looked up once per
// device, with that device current), or nullptr on a HIP error.
void* scratch_address() {
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  cache[dev].store(q, std::memory_order_release);
  return q;
}

int device_cus(int32_t* out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLAV_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return MLAV_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return MLAV_ERR_HIP;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return MLAV_OK;
}

int check_options(const mlav_options* opt) {
  if (!opt) return MLAV_OK;
  if (opt->nsplit < 0 || opt->pv_mode < 0 || opt->pv_mode > 1 || opt->kernel < 0 ||
      opt->kernel > 1 || opt->partials < 0 || opt->partials > 1 || opt->phase < 0 || opt->phase > 2 ||
      opt->merge < 0 || opt->merge > 1)
    return MLAV_ERR_ARG;
  return MLAV_OK;
}

bool compact_partials(const mlav_options* opt) {
  // the VALU cross-check kernel writes fp32 partials only
  return (opt ? opt->partials : 0) == 0 && (opt ? opt->kernel : 0) == 0;
}

// Row blocks of one sequence: its q * heads (token, head) rows in blocks of 64.
int32_t row_blocks(int32_t q, int32_t heads) { return (q * heads + kRows - 1) / kRows; }

int64_t round_chunk(int64_t c) {
  c = (c + kChunkGran - 1) / kChunkGran * kChunkGran;
  return c < kMinChunk ? kMinChunk : c;
}

// A workgroup's fixed cost (start-up loads, partial writes, its share of
// the combine) in tile steps, for the planner's estimates.
constexpr int64_t kFixedTiles = 12;

// Items of the batched chunk list dealt to one XCD in a row (one is a row
// block): runs of up to 8 row blocks of one chunk share its KV in an L2.
constexpr int32_t kListRun = 8;
int32_t list_run(int32_t nrb) { return nrb < kListRun ? nrb : kListRun; }

// Chunk length of a batched call, from the host copies of its total and
// longest lengths (the per-sequence lengths stay on the device).
//  - Unequal lengths: about two workgroups per CU over the whole batch (the
//    chunk list, long chunks first, evens out the different lengths; fewer,
//    longer chunks leave the last round unbalanced, more, shorter ones pay
//    the fixed cost more often). Below kSmallChunk keys per chunk the fixed
//    cost dominates, and the estimate below decides, up to kSmallChunk.
//  - Equal lengths (total = batch x max): every chunk is alike; of the
//    candidates (the longest sequence cut into 1, 2, 3, ... chunks), the one
//    whose workgroups fill the CUs in the fewest tile steps, each workgroup
//    paying its fixed cost.
// Estimate for unequal lengths, in tile steps of one CU: the total work
// spread over the CUs, with every workgroup's fixed cost (the chunks number
// about total / chunk + batch / 2), plus half a workgroup of tail; at least
// one whole workgroup.
constexpr int64_t kSmallChunk = 256;
int64_t batched_chunk(int64_t nrb, int32_t batch, int64_t total_kv, int64_t max_kv, int32_t num_cus) {
  const bool equal = total_kv == (int64_t)batch * max_kv;
  const int64_t cmax = round_chunk(max_kv);
  if (!equal) {
    const int64_t c = round_chunk((nrb * total_kv + 2 * (int64_t)num_cus - 1) / (2 * (int64_t)num_cus));
    if (c >= kSmallChunk) return c < cmax ? c : cmax;
  }
  const int64_t cus_per_xcd = num_cus >= kXcds ? num_cus / kXcds : 1;
  const double work = (double)nrb * ((double)total_kv / kTile);  // tile steps of the whole batch
  int64_t best = cmax, prev = -1;
  double best_cost = -1.0;
  for (int64_t ns = 1; ns <= 4096; ++ns) {
    const int64_t c = round_chunk((max_kv + ns - 1) / ns);
    if (c == prev) continue;
    prev = c;
    const double item = (double)((c + kTile - 1) / kTile + kFixedTiles);
    double cost;
    if (equal) {
      const int64_t items = nrb * batch * ((max_kv + c - 1) / c);
      const int64_t rounds = ((items + kXcds - 1) / kXcds + cus_per_xcd - 1) / cus_per_xcd;
      cost = (double)rounds * item;
    } else {
      const double chunks = (double)total_kv / (double)c + 0.5 * batch;
      cost = (work + (double)nrb * chunks * kFixedTiles) / num_cus + 0.5 * item;
      if (cost < item) cost = item;
    }
    if (best_cost < 0.0 || cost < best_cost) {
      best_cost = cost;
      best = c;
    }
    if (c <= kMinChunk) break;
  }
  if (!equal && best > kSmallChunk) best = kSmallChunk < cmax ? kSmallChunk : cmax;
  return best;
}

// Batched calls with unequal lengths run through the chunk list; equal
// lengths keep the (sequence, split, row block) order in one range per XCD,
// which has no empty items then.
bool chunk_list(int32_t batch, int64_t total_kv, int64_t max_kv) {
  return batch > 1 && total_kv != (int64_t)batch * max_kv;
}

// Grid of a batched call: covers the chunk list of any offsets that meet the
// contract (non-decreasing from 0 to total_kv, so that the chunks number at
// most ceil(total_kv / chunk) + batch - 1), dealt in runs of list_run(nrb).
int64_t list_grid(int64_t nrb, int32_t batch, int64_t total_kv, int64_t chunk, int64_t ns) {
  int64_t mcap = (total_kv + chunk - 1) / chunk + batch - 1;
  if (mcap > (int64_t)batch * ns) mcap = (int64_t)batch * ns;
  const int64_t run = list_run((int32_t)nrb);
  const int64_t runs = (mcap * nrb + run - 1) / run;
  return (runs + kXcds - 1) / kXcds * kXcds * run;
}

// One launch covers at most 2^32 - 1 work items (the dispatch packet's grid
// size is 32 bits): larger plans are refused before anything is launched.
constexpr int64_t kMaxLaunchItems = 0xffffffffll;

// Workgroups of the split phase for `nwork` (sequence, row block, split)
// items: the MFMA kernel rounds up to whole XCD rounds, the VALU kernel takes
// 16 workgroups per item.
int64_t split_grid(int kernel, int64_t nwork) {
  return kernel == 0 ? (nwork + kXcds - 1) / kXcds * kXcds : nwork * 16;
}

// Work items of the combine launch (launch() below): int16 partials take one
// 64-thread unit per (sequence, row block, 16-dim pair, row half), or one
// 256-thread workgroup per unit beyond 32 splits; fp32 partials take a
// 256-thread workgroup per two rows.
int64_t combine_items(int64_t batch, int64_t nrb, int64_t rows, int64_t nsplit, bool compact) {
  if (compact) return batch * nrb * 64 * (nsplit <= 32 ? 64 : kThreads);
  return (rows + 1) / 2 * kThreads;
}

int plan_impl(int32_t q, int32_t heads, int32_t batch, int64_t total_kv, int64_t max_kv,
              int32_t num_cus, const mlav_options* opt, mlav_plan* p) {
  if (q < 1 || q > MLAV_MAX_Q || batch < 1 || heads < 1 || heads > MLAV_MAX_HEADS) return MLAV_ERR_SHAPE;
  if (max_kv < q || total_kv < (int64_t)batch * q || max_kv > total_kv) return MLAV_ERR_SHAPE;
  if (max_kv > MLAV_MAX_KV) return MLAV_ERR_SHAPE;
  if (num_cus < 1) return MLAV_ERR_ARG;
  const int rc = check_options(opt);
  if (rc != MLAV_OK) return rc;
  const int64_t blocks = (int64_t)batch * row_blocks(q, heads);  // row blocks of the whole call
  int64_t chunk;
  if (opt && opt->nsplit > 0) {
    chunk = (max_kv + opt->nsplit - 1) / opt->nsplit;
    chunk = (chunk + kChunkGran - 1) / kChunkGran * kChunkGran;
  } else if (batch > 1) {
    chunk = batched_chunk(row_blocks(q, heads), batch, total_kv, max_kv, num_cus);
  } else {
    // one resident workgroup per CU: aim for about num_cus workgroups in total
    int64_t s_avg = num_cus / blocks;
    if (s_avg < 1) s_avg = 1;
    const int64_t avg_kv = (total_kv + batch - 1) / batch;
    chunk = (avg_kv + s_avg - 1) / s_avg;
    chunk = (chunk + kChunkGran - 1) / kChunkGran * kChunkGran;
    if (chunk < kMinChunk) chunk = kMinChunk;
  }
  const int64_t ns = (max_kv + chunk - 1) / chunk;
  const int64_t nwork = blocks * ns;
  if (nwork > (int64_t(1) << 30)) return MLAV_ERR_SHAPE;
  const int kernel = opt ? opt->kernel : 0;
  const int64_t grid = kernel == 0 && chunk_list(batch, total_kv, max_kv)
                           ? list_grid(row_blocks(q, heads), batch, total_kv, chunk, ns)
                           : split_grid(kernel, nwork);
  // merge = 1, 2..kMaxFusedSplits splits and int16 partials: the split kernel
  // merges them itself (one launch); otherwise the combine kernel runs
  const bool fused = ns >= 2 && ns <= kMaxFusedSplits && compact_partials(opt) && (opt ? opt->merge : 0) == 1;
  const int combine = ns > 1 ? (fused ? 2 : 1) : 0;
  if (grid * kThreads > kMaxLaunchItems) return MLAV_ERR_SHAPE;
  if (combine == 1 && combine_items(batch, row_blocks(q, heads), (int64_t)batch * q * heads, ns,
                                    compact_partials(opt)) > kMaxLaunchItems)
    return MLAV_ERR_SHAPE;
  p->nsplit = (int32_t)ns;
  p->tile = kTile;
  p->chunk = chunk;
  p->grid = (int32_t)grid;
  p->combine = combine;
  return MLAV_OK;
}

// Split partials in the workspace: values, then lse, then (compact only) the
// per-row scales, over [B, S, nrb * 64] rows (each sequence's q * heads rows
// padded to whole row blocks). Compact values are int16: 1024 bytes per row.
// A plan merged in the split kernel adds one 8-byte ticket per row block.

size_t workspace_bytes_for(const mlav_plan& p, int32_t q, int32_t heads, int32_t batch, bool compact) {
  if (!p.combine) return 0;
  const size_t rows = (size_t)batch * p.nsplit * row_blocks(q, heads) * kRows;
  const size_t tickets = p.combine == 2 ? (size_t)batch * row_blocks(q, heads) * sizeof(uint64_t) : 0;
  return compact ? rows * (kDl * sizeof(int16_t) + 2 * sizeof(float)) + tickets : rows * (kDl + 1) * sizeof(float);
}

// A fresh ticket epoch per call: 48 bits of a splitmix64 hash of a
// process-wide counter, so a stale word in the workspace (old partial values,
// another call's tickets) matches it with probability about 2^-48.
uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{0};
  uint64_t z = counter.fetch_add(1, std::memory_order_relaxed) + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z = (z ^ (z >> 31)) & ((uint64_t(1) << 48) - 1);
  return z ? z : 1;
}

// Points the partial pointers of `a` into the workspace (layout above).
void set_partials(Args& a, void* workspace, const mlav_plan& p, int32_t q, int32_t heads, int32_t batch,
                  bool compact) {
  const size_t rows = (size_t)batch * p.nsplit * row_blocks(q, heads) * kRows;
  a.part_o = nullptr;
  a.part_q = nullptr;
  a.part_scale = nullptr;
  a.part_lse = nullptr;
  a.tickets = nullptr;
  a.epoch = 0;
  if (!p.combine) return;
  if (compact) {
    a.part_q = (int16_t*)workspace;
    a.part_lse = (float*)(a.part_q + rows * kDl);
    a.part_scale = a.part_lse + rows;
    if (p.combine == 2) {
      a.tickets = (unsigned long long*)(a.part_scale + rows);  // rows is a multiple of 64: 8-byte aligned
      a.epoch = next_epoch();
    }
  } else {
    a.part_o = (float*)workspace;
    a.part_lse = a.part_o + rows * kDl;
  }
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

int launch(const Args& base, const mlav_plan& p, const mlav_options* opt, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  Args a = base;
  a.nsplit = p.nsplit;
  a.chunk = p.chunk;
  a.nrb = row_blocks(a.q, a.heads);
  a.nwork = a.batch * a.nrb * p.nsplit;
  a.per_xcd = (a.nwork + kXcds - 1) / kXcds;
  a.fixed_ns = 0;
  const int kernel = opt ? opt->kernel : 0;
  a.list_run = kernel == 0 && chunk_list(a.batch, a.total_kv, a.max_kv) ? list_run(a.nrb) : 0;
  const int pv_mode = opt ? opt->pv_mode : 0;
  const bool compact = a.part_q != nullptr;
  const int phase = opt ? opt->phase : 0;
  if (phase == 2) goto merge;
  if (kernel == 0) {
    // one instantiation per (weight form, partial format, KV layout)
    using K = void (*)(Args);
    static const K table[2][2][2] = {
        {{split_mfma_kernel<true, false, false, false>, split_mfma_kernel<true, false, true, false>},
         {split_mfma_kernel<true, true, false, false>, split_mfma_kernel<true, true, true, false>}},
        {{split_mfma_kernel<false, false, false, false>, split_mfma_kernel<false, false, true, false>},
         {split_mfma_kernel<false, true, false, false>, split_mfma_kernel<false, true, true, false>}}};
    // merged in the split kernel: its own instantiations, so that the other
    // kernels carry none of its code
    static const K fused_table[2][2] = {
        {split_mfma_kernel<true, true, false, true>, split_mfma_kernel<true, true, true, true>},
        {split_mfma_kernel<false, true, false, true>, split_mfma_kernel<false, true, true, true>}};
    const K k = p.combine == 2 ? fused_table[pv_mode == 0 ? 0 : 1][a.idx ? 1 : 0]
                               : table[pv_mode == 0 ? 0 : 1][compact ? 1 : 0][a.idx ? 1 : 0];
    hipLaunchKernelGGL(k, dim3(p.grid), dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL(split_valu_kernel, dim3(p.grid), dim3(kThreads), 0, st, a);
  }
  if (hipGetLastError() != hipSuccess) return MLAV_ERR_HIP;
  if (phase == 1) return MLAV_OK;
merge:
  if (p.combine == 1) {
    const int64_t rows = (int64_t)a.batch * a.q * a.heads;
    // compact partials: one unit per (sequence, row block, 16-dim pair, row half)
    const int64_t units = (int64_t)a.batch * a.nrb * 64;
    if (compact) {
      if (p.nsplit <= 32) {
        // loads per lane: the plan's split count rounded up to a multiple of 4
        using C = void (*)(Args, int64_t);
        static const C by_batch[8] = {combine_compact_kernel<4>,  combine_compact_kernel<8>,
                                      combine_compact_kernel<12>, combine_compact_kernel<16>,
                                      combine_compact_kernel<20>, combine_compact_kernel<24>,
                                      combine_compact_kernel<28>, combine_compact_kernel<32>};
        hipLaunchKernelGGL(by_batch[(p.nsplit + 3) / 4 - 1], dim3((unsigned)units), dim3(64), 0, st, a, units);
      } else {
        // loads per lane and batch: a wave's share of the splits, rounded up to a multiple of 4
        using C = void (*)(Args, int64_t);
        static const C by_batch[6] = {combine_compact_wide_kernel<12>, combine_compact_wide_kernel<16>,
                                      combine_compact_wide_kernel<20>, combine_compact_wide_kernel<24>,
                                      combine_compact_wide_kernel<28>, combine_compact_wide_kernel<32>};
        const int per_wave = (p.nsplit + 3) / 4;  // at least 9 here
        hipLaunchKernelGGL(by_batch[per_wave > 32 ? 5 : (per_wave + 3) / 4 - 3], dim3((unsigned)units),
                           dim3(kThreads), 0, st, a, units);
      }
    } else {
      hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((rows + 1) / 2)), dim3(kThreads), 0, st, a, rows);
    }
    if (hipGetLastError() != hipSuccess) return MLAV_ERR_HIP;
  }
  return MLAV_OK;
}

int common_checks(const void* qn, const void* qr, const void* lat, const void* rope,
                  const int32_t* parent, float scale, const float* out, const float* lse,
                  int32_t q, int32_t heads, const mlav_options* opt) {
  if (!qn || !qr || !lat || !rope || !parent || !out || !lse) return MLAV_ERR_NULL;
  if (q < 1 || q > MLAV_MAX_Q || heads < 1 || heads > MLAV_MAX_HEADS) return MLAV_ERR_SHAPE;
  if (!aligned(qn, 16) || !aligned(qr, 16) || !aligned(lat, 16) || !aligned(rope, 16) ||
      !aligned(out, 16) || !aligned(lse, 4) || !aligned(parent, 4))
    return MLAV_ERR_ALIGN;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MLAV_ERR_ARG;
  return check_options(opt);
}

}  // namespace mlav

using namespace mlav;

extern "C" {

int32_t mla_verify_plan(int32_t q_len, int32_t num_heads, int32_t batch, int64_t total_kv,
                        int64_t max_kv, int32_t num_cus, const mlav_options* opt,
                        mlav_plan* plan_out) {
  if (!plan_out) return MLAV_ERR_NULL;
  return plan_impl(q_len, num_heads, batch, total_kv, max_kv, num_cus, opt, plan_out);
}

size_t mla_verify_workspace_size(int32_t q_len, int32_t num_heads, int32_t batch, int64_t total_kv,
                                 int64_t max_kv, int32_t num_cus, const mlav_options* opt) {
  if (num_cus <= 0 && device_cus(&num_cus) != MLAV_OK) return 0;
  mlav_plan p;
  if (plan_impl(q_len, num_heads, batch, total_kv, max_kv, num_cus, opt, &p) != MLAV_OK) return 0;
  return workspace_bytes_for(p, q_len, num_heads, batch, compact_partials(opt));
}

}  // extern "C"

namespace mlav {

// One sequence: the body of mla_verify_ex and mla_verify_noalloc. With
// `scratch_call`, the workspace is the static scratch and a plan that needs
// more than it holds is refused with MLAV_ERR_SCRATCH.
int verify_single(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                  const void* k_rope, const int32_t* tree_parent, int64_t prefix_len, float scale,
                  float* out, float* lse, int32_t q_len, int32_t num_heads, void* workspace,
                  size_t workspace_bytes, void* stream, const mlav_options* opt, bool scratch_call) {
  int rc = common_checks(q_nope_absorbed, q_rope, kv_latent, k_rope, tree_parent, scale, out, lse,
                         q_len, num_heads, opt);
  if (rc != MLAV_OK) return rc;
  if (prefix_len < 0 || prefix_len + q_len > MLAV_MAX_KV) return MLAV_ERR_SHAPE;
  const int64_t n = prefix_len + q_len;
  int32_t cus = 0;
  rc = device_cus(&cus);
  if (rc != MLAV_OK) return rc;
  mlav_plan p;
  rc = plan_impl(q_len, num_heads, 1, n, n, cus, opt, &p);
  if (rc != MLAV_OK) return rc;
  const bool compact = compact_partials(opt);
  const size_t need = workspace_bytes_for(p, q_len, num_heads, 1, compact);
  if (scratch_call) {
    if (need > MLAV_SCRATCH_BYTES) return MLAV_ERR_SCRATCH;
    if (need > 0) {
      workspace = scratch_address();
      if (!workspace) return MLAV_ERR_HIP;
      workspace_bytes = MLAV_SCRATCH_BYTES;
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLAV_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return MLAV_ERR_ALIGN;
  Args a{};
  a.qn = (const uint16_t*)q_nope_absorbed;
  a.qr = (const uint16_t*)q_rope;
  a.lat = (const uint16_t*)kv_latent;
  a.rope = (const uint16_t*)k_rope;
  a.parent = tree_parent;
  a.offs = nullptr;
  a.out = out;
  a.lse = lse;
  set_partials(a, workspace, p, q_len, num_heads, 1, compact);
  a.single_n = n;
  a.total_kv = n;
  a.max_kv = n;
  a.scale_log2 = scale * kLog2e;
  a.q = q_len;
  a.heads = num_heads;
  a.batch = 1;
  return launch(a, p, opt, stream);
}

}  // namespace mlav

extern "C" {

int32_t mla_verify_ex(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                      const void* k_rope, const int32_t* tree_parent, int64_t prefix_len,
                      float scale, float* out, float* lse, int32_t q_len, int32_t num_heads,
                      void* workspace, size_t workspace_bytes, void* stream,
                      const mlav_options* opt) {
  return verify_single(q_nope_absorbed, q_rope, kv_latent, k_rope, tree_parent, prefix_len, scale, out,
                       lse, q_len, num_heads, workspace, workspace_bytes, stream, opt, false);
}

int32_t mla_verify_noalloc(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                           const void* k_rope, const int32_t* tree_parent, int64_t prefix_len,
                           float scale, float* out, float* lse, int32_t q_len, int32_t num_heads,
                           void* stream, const mlav_options* opt) {
  return verify_single(q_nope_absorbed, q_rope, kv_latent, k_rope, tree_parent, prefix_len, scale, out,
                       lse, q_len, num_heads, nullptr, 0, stream, opt, true);
}

int32_t mla_verify(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                   const void* k_rope, const int32_t* tree_parent, int64_t prefix_len, float scale,
                   float* out, float* lse, int32_t q_len, int32_t num_heads, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return mla_verify_ex(q_nope_absorbed, q_rope, kv_latent, k_rope, tree_parent, prefix_len, scale,
                       out, lse, q_len, num_heads, workspace, workspace_bytes, stream, nullptr);
}

int32_t mla_verify_batched(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                           const void* k_rope, const int32_t* tree_parent,
                           const int64_t* kv_offsets, int32_t batch, int64_t total_kv,
                           int64_t max_kv, float scale, float* out, float* lse, int32_t q_len,
                           int32_t num_heads, void* workspace, size_t workspace_bytes,
                           void* stream, const mlav_options* opt) {
  int rc = common_checks(q_nope_absorbed, q_rope, kv_latent, k_rope, tree_parent, scale, out, lse,
                         q_len, num_heads, opt);
  if (rc != MLAV_OK) return rc;
  if (!kv_offsets) return MLAV_ERR_NULL;
  if (!aligned(kv_offsets, 8)) return MLAV_ERR_ALIGN;
  if (batch < 1 || max_kv < q_len || total_kv < (int64_t)batch * q_len || max_kv > total_kv)
    return MLAV_ERR_SHAPE;
  int32_t cus = 0;
  rc = device_cus(&cus);
  if (rc != MLAV_OK) return rc;
  mlav_plan p;
  rc = plan_impl(q_len, num_heads, batch, total_kv, max_kv, cus, opt, &p);
  if (rc != MLAV_OK) return rc;
  const bool compact = compact_partials(opt);
  const size_t need = workspace_bytes_for(p, q_len, num_heads, batch, compact);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLAV_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return MLAV_ERR_ALIGN;
  Args a{};
  a.qn = (const uint16_t*)q_nope_absorbed;
  a.qr = (const uint16_t*)q_rope;
  a.lat = (const uint16_t*)kv_latent;
  a.rope = (const uint16_t*)k_rope;
  a.parent = tree_parent;
  a.offs = kv_offsets;
  a.out = out;
  a.lse = lse;
  set_partials(a, workspace, p, q_len, num_heads, batch, compact);
  a.single_n = 0;
  a.total_kv = total_kv;
  a.max_kv = max_kv;
  a.scale_log2 = scale * kLog2e;
  a.q = q_len;
  a.heads = num_heads;
  a.batch = batch;
  return launch(a, p, opt, stream);
}

int32_t mla_verify_paged(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                         const void* k_rope, const int32_t* kv_index, int64_t pool_rows,
                         const int32_t* tree_parent, const int64_t* kv_offsets, int32_t batch,
                         int64_t total_kv, int64_t max_kv, float scale, float* out, float* lse,
                         int32_t q_len, int32_t num_heads, void* workspace, size_t workspace_bytes,
                         void* stream, const mlav_options* opt) {
  int rc = common_checks(q_nope_absorbed, q_rope, kv_latent, k_rope, tree_parent, scale, out, lse,
                         q_len, num_heads, opt);
  if (rc != MLAV_OK) return rc;
  if (!kv_index) return MLAV_ERR_NULL;
  if (!aligned(kv_index, 4)) return MLAV_ERR_ALIGN;
  if (pool_rows < 1 || pool_rows > MLAV_MAX_POOL) return MLAV_ERR_SHAPE;
  if (batch < 1 || max_kv < q_len || total_kv < (int64_t)batch * q_len || max_kv > total_kv)
    return MLAV_ERR_SHAPE;
  if (kv_offsets) {
    if (!aligned(kv_offsets, 8)) return MLAV_ERR_ALIGN;
  } else if (batch != 1 || max_kv != total_kv) {
    return MLAV_ERR_ARG;  // without offsets there is one sequence of total_kv rows
  }
  int32_t cus = 0;
  rc = device_cus(&cus);
  if (rc != MLAV_OK) return rc;
  mlav_plan p;
  rc = plan_impl(q_len, num_heads, batch, total_kv, max_kv, cus, opt, &p);
  if (rc != MLAV_OK) return rc;
  const bool compact = compact_partials(opt);
  const size_t need = workspace_bytes_for(p, q_len, num_heads, batch, compact);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLAV_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return MLAV_ERR_ALIGN;
  Args a{};
  a.qn = (const uint16_t*)q_nope_absorbed;
  a.qr = (const uint16_t*)q_rope;
  a.lat = (const uint16_t*)kv_latent;
  a.rope = (const uint16_t*)k_rope;
  a.parent = tree_parent;
  a.offs = kv_offsets;
  a.idx = kv_index;
  a.pool_rows = pool_rows;
  a.out = out;
  a.lse = lse;
  set_partials(a, workspace, p, q_len, num_heads, batch, compact);
  a.single_n = kv_offsets ? 0 : total_kv;
  a.total_kv = total_kv;
  a.max_kv = max_kv;
  a.scale_log2 = scale * kLog2e;
  a.q = q_len;
  a.heads = num_heads;
  a.batch = batch;
  return launch(a, p, opt, stream);
}

int32_t mla_verify_partials(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                            const void* k_rope, const int32_t* tree_parent, int64_t prefix_len,
                            float scale, float* part_out, float* part_lse, int32_t q_len,
                            int32_t num_heads, const mlav_plan* plan, void* stream,
                            const mlav_options* opt) {
  int rc = common_checks(q_nope_absorbed, q_rope, kv_latent, k_rope, tree_parent, scale, part_out,
                         part_lse, q_len, num_heads, opt);
  if (rc != MLAV_OK) return rc;
  if (!plan) return MLAV_ERR_NULL;
  if (prefix_len < 0 || prefix_len + q_len > MLAV_MAX_KV) return MLAV_ERR_SHAPE;
  const int64_t n = prefix_len + q_len;
  // the kernels take the chunk as a 32-bit key count: a chunk longer than any
  // sequence is refused rather than narrowed
  if (plan->tile != kTile || plan->chunk < kTile || plan->chunk > MLAV_MAX_KV || plan->chunk % kTile != 0 ||
      plan->nsplit < 1 || plan->nsplit != (n + plan->chunk - 1) / plan->chunk)
    return MLAV_ERR_ARG;
  mlav_plan p = *plan;
  const int kernel = opt ? opt->kernel : 0;
  const int64_t grid = split_grid(kernel, (int64_t)row_blocks(q_len, num_heads) * p.nsplit);
  if (grid * kThreads > kMaxLaunchItems) return MLAV_ERR_SHAPE;
  p.grid = (int32_t)grid;
  p.combine = 0;
  Args a{};
  a.qn = (const uint16_t*)q_nope_absorbed;
  a.qr = (const uint16_t*)q_rope;
  a.lat = (const uint16_t*)kv_latent;
  a.rope = (const uint16_t*)k_rope;
  a.parent = tree_parent;
  a.offs = nullptr;
  // with one split the partial is the final result; the layouts coincide
  a.out = part_out;
  a.lse = part_lse;
  a.part_o = part_out;
  a.part_lse = part_lse;
  a.single_n = n;
  a.total_kv = n;
  a.max_kv = n;
  a.scale_log2 = scale * kLog2e;
  a.q = q_len;
  a.heads = num_heads;
  a.batch = 1;
  return launch(a, p, opt, stream);
}

int32_t mla_verify_check_tree(const int32_t* host_parent, int32_t q_len) {
  if (!host_parent) return MLAV_ERR_NULL;
  if (q_len < 1 || q_len > MLAV_MAX_Q) return MLAV_ERR_SHAPE;
  for (int32_t i = 0; i < q_len; ++i)
    if (!(host_parent[i] == -1 || (host_parent[i] >= 0 && host_parent[i] < i))) return MLAV_ERR_TREE;
  return MLAV_OK;
}

int32_t mla_verify_combine(const float* part_out, const float* part_lse, int32_t nsplit,
                           int64_t rows, float* out, float* lse, void* stream) {
  if (!part_out || !part_lse || !out || !lse) return MLAV_ERR_NULL;
  // two rows per 256-thread workgroup: rows * 128 work items must stay below 2^32
  if (nsplit < 1 || rows < 1 || rows > MLAV_MAX_COMBINE_ROWS) return MLAV_ERR_SHAPE;
  if (!aligned(part_out, 16) || !aligned(out, 16) || !aligned(part_lse, 4) || !aligned(lse, 4))
    return MLAV_ERR_ALIGN;
  if (rows % kRows != 0) return MLAV_ERR_SHAPE;  // whole row blocks (padded partial layout)
  Args a{};
  a.part_o = const_cast<float*>(part_out);
  a.part_lse = const_cast<float*>(part_lse);
  a.out = out;
  a.lse = lse;
  a.q = (int32_t)(rows / kRows);  // one block of 64 rows per "token"
  a.heads = kRows;
  a.nrb = a.q;
  a.batch = 1;
  a.nsplit = nsplit;
  a.fixed_ns = nsplit;
  a.chunk = 1;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((rows + 1) / 2)), dim3(kThreads), 0,
                     (hipStream_t)stream, a, rows);
  return hipGetLastError() == hipSuccess ? MLAV_OK : MLAV_ERR_HIP;
}

const char* mla_verify_strerror(int32_t status) {
  switch (status) {
    case MLAV_OK: return "ok";
    case MLAV_ERR_NULL: return "a required pointer is NULL";
    case MLAV_ERR_SHAPE: return "a size is out of range";
    case MLAV_ERR_TREE: return "tree_parent is not topologically ordered";
    case MLAV_ERR_ALIGN: return "a pointer is not aligned (16 B for tensors, 4 B for lse/parents)";
    case MLAV_ERR_WORKSPACE: return "workspace missing or too small";
    case MLAV_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLAV_ERR_HIP: return "HIP runtime error";
    case MLAV_ERR_ARG: return "invalid scalar or option value";
    case MLAV_ERR_SCRATCH: return "the call needs more than the static scratch (MLAV_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
