/*
 * mla_verify.h -- C ABI of the MI355X (gfx950) MLA tree-verify attention library.
 *
 * The operation is absorbed-form Multi-head Latent Attention for the verify
 * step of tree speculative decoding: every draft-tree token's query heads
 * attend over the shared compressed KV cache plus the tree's own tokens under
 * an ancestor mask. (Page "The Flash Attention Kernel That Had to Be Built:
 * Designing sm_120 MLA Verify", sections "Strategic Context" and "What Input
 * Knowledge Is Required": 512-d latent kv_c plus a 64-d decoupled rope key per
 * cached token, absorbed q_nope plus q_pe per query head, masked positions set
 * to -inf before the softmax. Page "The Moment of Truth", benchmark table
 * header: H=64, Dl=512, Dr=64.)
 *
 *   s[i,h,j]  = scale * (q_nope[i,h,:] . kv_latent[j,:] + q_rope[i,h,:] . k_rope[j,:])
 *   visible   = j < P  or  (j - P) is i itself or an ancestor of i in the tree
 *   out[i,h]  = softmax_j(s[i,h,visible]) @ kv_latent[visible]     (fp32)
 *   lse[i,h]  = ln sum_j exp(s[i,h,j])  over the visible keys     (fp32, natural log)
 *
 * The KV is split into chunks processed by separate workgroups (flash-decode
 * partials) and a second kernel merges them with the log-sum-exp combine
 * (page "The Decisive Microbench", section "The KV-Split Solution").
 *
 * Conventions for every entry point below:
 *  - bf16 tensors are passed as raw 16-bit patterns (const void*), row-major
 *    and contiguous; fp32 outputs likewise. All tensor pointers are DEVICE
 *    pointers unless a name says host.
 *  - KV layout per sequence: rows [0, P) are the cached prefix, rows
 *    [P, P+q) are the q draft-tree tokens in node order (node t at row P+t).
 *  - tree_parent[i] is -1 (a child of the last committed prefix token) or an
 *    earlier node index in [0, i). Each token sees itself and its ancestors.
 *  - The caller owns every buffer. The library allocates no device memory and
 *    keeps no pointer after a call returns. Inputs are read only; out and lse
 *    are fully overwritten. Aliasing between inputs, outputs and workspace is
 *    undefined behaviour.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream): no host synchronisation, no allocation and no device-to-host
 *    copy happen inside, so a call can be captured into a HIP graph.
 *  - Arguments are validated on the host before anything is launched; on an
 *    error nothing is launched and a status code is returned. The device-side
 *    contents (the tree, the offsets) are a documented precondition; the
 *    kernels stay in bounds for any tree (the ancestor walk is bounded by q)
 *    and write NaN for a sequence whose offsets are inconsistent.
 *  - Launch failures return MLAV_ERR_HIP; faults inside a kernel surface at the
 *    caller's next synchronisation.
 *  - Numeric range (a precondition the host cannot check without reading the
 *    device data): every score s[i,h,j] and every partial 576-term dot product
 *    must be finite in fp32, and |kv_latent| < 2^31 (about 2.1e9). Under these
 *    the results are finite: inside a chunk the softmax weights stay at most
 *    2^96 relative to a fixed reference, a chunk whose scores climb past that
 *    or whose fp32 accumulators overflow is redone once with the chunk's own
 *    maximum as the reference (weights at most 1), and below 2^31 no single
 *    weight x value product overflows.
 */
#ifndef MLA_VERIFY_H
#define MLA_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MLAV_OK 0
#define MLAV_ERR_NULL 1        /* a required pointer is NULL */
#define MLAV_ERR_SHAPE 2       /* a size is out of range */
#define MLAV_ERR_TREE 3        /* tree_parent is not topologically ordered (host check) */
#define MLAV_ERR_ALIGN 4       /* a tensor pointer is not 16-byte aligned (lse and parents: 4) */
#define MLAV_ERR_WORKSPACE 5   /* workspace missing or smaller than mla_verify_workspace_size */
#define MLAV_ERR_UNSUPPORTED 6 /* a valid but unimplemented configuration */
#define MLAV_ERR_HIP 7         /* the HIP runtime reported an error */
#define MLAV_ERR_ARG 8         /* a scalar or option value is invalid */
#define MLAV_ERR_SCRATCH 9     /* mla_verify_noalloc: the call needs more than MLAV_SCRATCH_BYTES */

#define MLAV_MAX_Q 64    /* q_len limit: one 64-bit ancestor mask per token */
#define MLAV_ROWS 64     /* (token, head) rows per workgroup: one row block */
#define MLAV_MAX_HEADS 1024 /* num_heads limit */
#define MLAV_DL 512      /* latent width (value width) */
#define MLAV_DR 64       /* rope width */
#define MLAV_MAX_KV 4000000 /* KV rows per sequence (byte offsets into one sequence's
                               latent rows must stay below 2^32) */
#define MLAV_MAX_POOL 4000000 /* rows of a paged KV pool (byte offsets into the pool's
                                 latent rows must stay below 2^32) */
#define MLAV_MAX_COMBINE_ROWS (1 << 24) /* rows of one mla_verify_combine call */
#define MLAV_SCRATCH_BYTES (24u << 20) /* static device scratch of mla_verify_noalloc (24 MiB) */

/* Tuning knobs; a NULL options pointer means all zeros. */
typedef struct mlav_options {
  int32_t nsplit;  /* 0: the planner picks the KV split count; >0: request this many
                      splits (the planner rounds the chunk to whole tiles, so the
                      effective count can be lower) */
  int32_t pv_mode; /* 0: softmax weights enter the value product as a bf16 hi+lo
                      pair (about 16 significant bits, the default);
                      1: a single bf16 weight (8 bits; faster, looser) */
  int32_t kernel;  /* 0: bf16 MFMA kernel (default); 1: plain fp32 VALU kernel
                      (a slow second implementation kept for cross-checks) */
  int32_t partials; /* storage of the split partials between the two kernels of
                       mla_verify / _ex / _batched:
                       0: int16 values with one fp32 scale per (row, split)
                          (the default; each value is off by at most 2^-16 of
                          the largest |value| of its row, and the partial
                          traffic is half that of fp32);
                       1: fp32 values (the format mla_verify_partials writes) */
  int32_t phase;    /* 0: the whole call; 1: the split kernel only (with more than
                       one split the partials stay in the workspace); 2: the
                       combine kernel only, on the workspace that a phase-1 call
                       with the same arguments filled (nothing runs when the plan
                       has one split or is merged in the split kernel: phase 1
                       then wrote out and lse) */
  int32_t merge;    /* 0 (the default): plans with more than one split run the
                       combine kernel after the split kernel;
                       1: a plan of 2..4 splits with int16 partials (short
                       prefixes) is merged in the split kernel instead: the
                       last workgroup of each row block to finish merges that
                       block's splits, so the call is one launch
                       (plan->combine = 2; the workspace then also holds one
                       8-byte ticket per row block, which needs no clearing).
                       On MI355X this is slower than the two launches (one CU
                       pulls all partials of its row block, after two extra
                       device-scope round trips), hence not the default */
} mlav_options;

/* What the planner decided for one call. */
typedef struct mlav_plan {
  int32_t nsplit;  /* KV splits per sequence (of the longest sequence) */
  int32_t tile;    /* keys per wave tile */
  int64_t chunk;   /* keys per split (a multiple of tile) */
  int32_t grid;    /* workgroups of the split kernel */
  int32_t combine; /* 0: one split, the split kernel writes out and lse;
                      1: the combine kernel runs after the split kernel;
                      2: the split kernel merges the splits itself (see
                         mlav_options.merge) */
} mlav_plan;

/*
 * One sequence.
 *   q_nope_absorbed [q_len, num_heads, 512] bf16   absorbed nope query
 *   q_rope          [q_len, num_heads, 64]  bf16   rope query (RoPE already applied)
 *   kv_latent       [prefix_len + q_len, 512] bf16 latent keys = values
 *   k_rope          [prefix_len + q_len, 64]  bf16 rope keys
 *   tree_parent     [q_len] int32
 *   prefix_len      >= 0 cached tokens before the tree; prefix_len + q_len <= MLAV_MAX_KV
 *   scale           fp32 factor (> 0) on the whole 576-d dot product
 *   out             [q_len, num_heads, 512] fp32
 *   lse             [q_len, num_heads] fp32, natural log
 *   q_len           1 .. 64;  num_heads 1 .. MLAV_MAX_HEADS (any count: a workgroup
 *                   covers 64 consecutive (token, head) rows, so several tokens
 *                   share one at num_heads < 64 and a token spans several at
 *                   num_heads > 64)
 *   workspace       device scratch of at least mla_verify_workspace_size(...)
 *                   bytes (may be NULL when that size is 0)
 */
int32_t mla_verify(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                   const void* k_rope, const int32_t* tree_parent, int64_t prefix_len, float scale,
                   float* out, float* lse, int32_t q_len, int32_t num_heads, void* workspace,
                   size_t workspace_bytes, void* stream);

/* mla_verify with explicit options (NULL = defaults). */
int32_t mla_verify_ex(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                      const void* k_rope, const int32_t* tree_parent, int64_t prefix_len,
                      float scale, float* out, float* lse, int32_t q_len, int32_t num_heads,
                      void* workspace, size_t workspace_bytes, void* stream,
                      const mlav_options* opt);

/*
 * mla_verify_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The split partials live in a static device array of MLAV_SCRATCH_BYTES
 * that the library holds on each device it runs on until the process ends
 * (its address is looked up once per device, on the first call there, with
 * hipGetSymbolAddress). The call allocates nothing and calls no allocating
 * routine; the caller still passes inputs and outputs. A call whose plan
 * needs more partial storage than MLAV_SCRATCH_BYTES returns MLAV_ERR_SCRATCH
 * and launches nothing: every plan the library makes by itself for one
 * sequence with int16 partials fits (at most one workgroup per CU, 66 KB of
 * partials each, about 17 MB on 256 CUs); forced large split counts or fp32
 * partials may not. Every call on one device shares that device's array:
 * calls that overlap on one device (two streams, two host threads) race and
 * give undefined results; calls in stream order are safe (the array keeps
 * the last call's contents, and nothing in it needs clearing). Arguments,
 * options and errors otherwise as mla_verify_ex.
 */
int32_t mla_verify_noalloc(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                           const void* k_rope, const int32_t* tree_parent, int64_t prefix_len,
                           float scale, float* out, float* lse, int32_t q_len, int32_t num_heads,
                           void* stream, const mlav_options* opt);

/*
 * Several sequences in one call: the pages' grid spans the batch as well as
 * the query positions, head groups and KV splits (page "The Decisive
 * Microbench", section "The KV-Split Solution"; page "The Moment of Truth",
 * section "The Analysis: Occupancy Starvation", one block per batch entry,
 * query position and head tile). Ragged prefixes are stored back to back with
 * an offsets array (this library's layout; the pages benchmark one stream).
 * batch independent sequences sharing q_len; sequence b owns KV rows
 * [kv_offsets[b], kv_offsets[b+1]) (its prefix then its q_len tree tokens).
 *   q_nope_absorbed [batch, q_len, num_heads, 512], q_rope [batch, q_len, num_heads, 64]
 *   kv_latent [total_kv, 512], k_rope [total_kv, 64], tree_parent [batch, q_len]
 *   kv_offsets [batch + 1] int64 DEVICE array, non-decreasing, kv_offsets[0] = 0
 *   total_kv = kv_offsets[batch], max_kv = max_b (kv_offsets[b+1] - kv_offsets[b]):
 *   host copies of two device facts, used for planning and bounds checks
 *   out [batch, q_len, num_heads, 512], lse [batch, q_len, num_heads]
 * Scheduling: sequences of unequal lengths run through a list of their KV
 * chunks that the split kernel builds from kv_offsets (full chunks first,
 * then each sequence's shorter last chunk, longest first), so that the work
 * spreads over the CUs whatever the mix of lengths; equal lengths keep one
 * range of (sequence, split, row block) items per XCD. The grid covers the
 * chunks of any offsets that meet the contract above. A sequence whose own
 * bounds are inconsistent (start below 0, end past total_kv, length below
 * q_len or above max_kv) gets NaN rows. If the offsets are not
 * non-decreasing, the other sequences are exact as long as their chunks fit
 * that grid; past it, their rows are unspecified (never out of bounds).
 */
int32_t mla_verify_batched(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                           const void* k_rope, const int32_t* tree_parent,
                           const int64_t* kv_offsets, int32_t batch, int64_t total_kv,
                           int64_t max_kv, float scale, float* out, float* lse, int32_t q_len,
                           int32_t num_heads, void* workspace, size_t workspace_bytes,
                           void* stream, const mlav_options* opt);

/*
 * Paged KV with one token per page (the layout of a serving KV pool whose
 * page size is 1: page "The Moment of Truth", section "Output Knowledge
 * Created", and page "The Validation Milestone", the Triton-baseline
 * paragraph, where it makes the attention a scattered gather). The keys and
 * values live in a pool of pool_rows rows, and a page table maps each
 * sequence's logical KV rows (its prefix, then its q_len tree tokens) to pool
 * rows; otherwise the operation is the one above.
 *   kv_latent [pool_rows, 512], k_rope [pool_rows, 64] bf16   the pool
 *   kv_index  [total_kv] int32 DEVICE: logical row -> pool row; an entry
 *             outside [0, pool_rows) reads as a row of zeros (never out of
 *             bounds)
 *   pool_rows 1 .. MLAV_MAX_POOL
 *   kv_offsets [batch + 1] int64 DEVICE: sequence b owns logical rows
 *             [kv_offsets[b], kv_offsets[b+1]) of kv_index; may be NULL for a
 *             single sequence (batch = 1, max_kv = total_kv = its row count)
 *   q_nope_absorbed, q_rope, tree_parent, out, lse: as mla_verify_batched
 * The page-table entries are read on the device; the kernels stay in bounds
 * for any entries. Workspace: as mla_verify_batched.
 */
int32_t mla_verify_paged(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                         const void* k_rope, const int32_t* kv_index, int64_t pool_rows,
                         const int32_t* tree_parent, const int64_t* kv_offsets, int32_t batch,
                         int64_t total_kv, int64_t max_kv, float scale, float* out, float* lse,
                         int32_t q_len, int32_t num_heads, void* workspace, size_t workspace_bytes,
                         void* stream, const mlav_options* opt);

/* Workspace bytes a call with these sizes and options needs (0 when no split
   is needed): the scratch where each KV split leaves its partial result and
   statistics for the merge (page "The Decisive Microbench", section "The
   KV-Split Solution"). It depends on opt->partials.
   num_cus = 0 queries the current HIP device; pass the CU count to plan
   without a device. For one sequence use batch = 1 and
   total_kv = max_kv = prefix_len + q_len. Returns 0 for invalid sizes. */
size_t mla_verify_workspace_size(int32_t q_len, int32_t num_heads, int32_t batch, int64_t total_kv,
                                 int64_t max_kv, int32_t num_cus, const mlav_options* opt);

/* The planner as a pure host function (no HIP call): the split count and the
   chunk length, chosen so that the (sequence, row block, split) work items
   fill the GPU's CUs at short prefixes as well as long ones (page "The
   Decisive Microbench", section "The KV-Split Solution": partitioning the KV
   across blocks so that enough blocks exist to keep every SM busy; page "The
   Validation Milestone", section "The Problem: Occupancy Starvation").
   One sequence: about num_cus work items. A batch of equal lengths (total_kv
   = batch x max_kv): the split count whose items fill the CUs in the fewest
   tile steps. Unequal lengths: about two items per CU over the batch (a
   fixed-cost estimate below 256 keys per chunk); plan_out->grid then covers
   the kernel's list of every sequence's chunks (mla_verify_batched).
   Returns MLAV_ERR_SHAPE for sizes out of range (also for a plan whose
   split or combine launch would exceed 2^32 - 1 threads), MLAV_ERR_ARG for
   num_cus < 1 or invalid options; plan_out is written only on MLAV_OK. */
int32_t mla_verify_plan(int32_t q_len, int32_t num_heads, int32_t batch, int64_t total_kv,
                        int64_t max_kv, int32_t num_cus, const mlav_options* opt,
                        mlav_plan* plan_out);

/*
 * The split phase alone, for a caller-chosen plan (from mla_verify_plan):
 * each KV chunk of plan->chunk keys yields a normalised partial output and its
 * lse (the "unnormalised accumulator and statistics" of each split, page "The
 * Decisive Microbench", section "The KV-Split Solution", here stored
 * normalised) in
 *   part_out [plan->nsplit, q_len, num_heads, 512] fp32 and
 *   part_lse [plan->nsplit, q_len, num_heads] fp32 (natural log).
 * mla_verify_combine(part_out, part_lse, plan->nsplit, q_len * num_heads, ...)
 * then gives exactly what mla_verify returns (for q_len * num_heads not a
 * multiple of 64 the rows are padded: part_out is [plan->nsplit, R, 512] with
 * R = q_len * num_heads rounded up to a multiple of 64, and the combine then
 * takes rows = R; the padding rows hold unspecified values). Partials from several callers
 * (e.g. KV shards) can be stacked and combined the same way; a split that sees
 * no visible key has lse = -inf and a zero output. The plan must satisfy
 * nsplit = ceil((prefix_len + q_len) / chunk) with chunk a positive multiple of
 * plan->tile (32) and at most MLAV_MAX_KV; otherwise MLAV_ERR_ARG. A plan
 * whose split launch would exceed 2^32 - 1 threads gives MLAV_ERR_SHAPE. Other
 * arguments as for mla_verify.
 */
int32_t mla_verify_partials(const void* q_nope_absorbed, const void* q_rope, const void* kv_latent,
                            const void* k_rope, const int32_t* tree_parent, int64_t prefix_len,
                            float scale, float* part_out, float* part_lse, int32_t q_len,
                            int32_t num_heads, const mlav_plan* plan, void* stream,
                            const mlav_options* opt);

/* Host-side check of a HOST copy of a tree: MLAV_OK or MLAV_ERR_TREE. */
int32_t mla_verify_check_tree(const int32_t* host_parent, int32_t q_len);

/* The combine kernel alone, on caller-made partials: the log-sum-exp merge of
   the split partials (page "The Decisive Microbench", section "The KV-Split
   Solution": a light second kernel merges the per-split results using their
   statistics).
   part_out [nsplit, rows, 512] fp32 (each normalised), part_lse [nsplit, rows]
   fp32 (natural log; -inf marks an empty part) -> out [rows, 512], lse [rows].
   rows must be a positive multiple of 64 (MLAV_ROWS: the padded row layout
   mla_verify_partials writes) and at most MLAV_MAX_COMBINE_ROWS; otherwise
   MLAV_ERR_SHAPE. nsplit >= 1. A row whose parts are all empty gets out = 0
   and lse = -inf. */
int32_t mla_verify_combine(const float* part_out, const float* part_lse, int32_t nsplit,
                           int64_t rows, float* out, float* lse, void* stream);

/* Human-readable text for a status code (static storage). */
const char* mla_verify_strerror(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_H */
