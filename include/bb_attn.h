/*
 * bb_attn.h -- C ABI of libbb_attn.so: BigBird block-sparse self-attention
 * forward on AMD Instinct MI355X (gfx950).
 *
 * The operation (page "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
 * section "BigBird：从二次方注意力到线性稀疏注意力"; paper card "Big Bird:
 * Transformers for Longer Sequences", section "方法适配"):
 *   Q, K, V are cut into blocks of `block` tokens, nb = L / block.  Query
 *   blocks 0 and nb-1 are global and attend every key.  A middle query block
 *   i (1 <= i <= nb-2) attends the band {i-1, i, i+1}, the two global key
 *   blocks and the r random blocks listed in rand_idx[h][i-1][:].  Logits are
 *   q.k / sqrt(d); keys marked as padding get -10000 added; one softmax per
 *   query row over all attended keys; out = softmax . V.
 *
 * Conventions for every function below:
 *   - Return value is a bb_status; nothing throws across the ABI.
 *   - All argument validation happens on the host before any HIP call.  On a
 *     validation error nothing is launched and no memory is touched.
 *   - The library never allocates or frees memory; the caller owns every
 *     buffer.  It keeps no mutable global state.
 *   - Tensors are dense, row-major, contiguous.
 */
#ifndef BB_ATTN_H_
#define BB_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BB_ABI_VERSION 1

typedef enum {
  BB_OK = 0,
  BB_ERR_NULL = 1,       /* a required pointer is NULL */
  BB_ERR_SHAPE = 2,      /* unsupported or inconsistent sizes */
  BB_ERR_DTYPE = 3,      /* dtype is not a bb_dtype value */
  BB_ERR_RAND_IDX = 4,   /* random-block table violates its constraints */
  BB_ERR_WORKSPACE = 5,  /* workspace smaller than bb_attn_workspace_bytes() */
  BB_ERR_HIP = 6,        /* a HIP launch reported an error */
  BB_ERR_ALIAS = 7,      /* out overlaps q, k or v */
  BB_ERR_ALIGN = 8       /* a device pointer is not aligned as documented */
} bb_status;

typedef enum { BB_FP32 = 0, BB_BF16 = 1 } bb_dtype;

/* Flags for bb_attn_forward_ex.  One launch mode, optionally one phase. */
#define BB_LAUNCH_FUSED 0u /* global-row and middle-block work units share one grid, then the split-K merge */
#define BB_LAUNCH_SPLIT 1u /* global-row kernel, middle-block kernel, split-K merge: three launches */
#define BB_PHASE_UNITS 2u  /* enqueue only the work-unit launch(es); the output rows of the two
                              global blocks are not written yet */
#define BB_PHASE_MERGE 4u  /* enqueue only the split-K merge that writes the global rows; it must
                              follow a BB_PHASE_UNITS call with the same arguments and workspace
                              on the same stream */
                           /* neither phase bit, or both: the whole forward */
#define BB_QUERY_MASK 8u   /* pair masking: an attended pair gets the -10000 offset when its query
                              or its key is padding (default: when its key is).  Page "models 仓库中的
                              BigBird：线性复杂度稀疏注意力与长序列训练的完整实践", section
                              "随机块掩码是如何生成的": the layer receives the blocked mask and a band mask
                              built from it by an einsum of the query and key sides.  Rows of valid
                              queries are unchanged; a padded query row has the same offset on every
                              pair, which cancels in its softmax: it is the unmasked attention row.
                              No effect when pad_mask is NULL.  Also taken by
                              bb_attn_forward_lse_ex and bb_attn_backward_ex (give both the flag,
                              or neither). */
#define BB_ORDINARY_UNITS 16u /* run the ordinary work units even for a small problem.  By default,
                              when the ordinary units are too few to fill the device (fewer than
                              512 of 64 query rows), the fp32 kernels and the bf16 kernels of block
                              64 split every query block over its key tiles instead and merge the
                              chunks afterwards (BB_LAUNCH_SPLIT then has no second launch); the
                              result agrees to rounding.  The backward (bb_attn_backward_ex, any
                              dtype and block) splits the same way: every query block over its
                              key tiles for dQ, every key block over its query tiles for dK and
                              dV, summed afterwards.  For tests that want the ordinary units. */

/* Version of this ABI (BB_ABI_VERSION of the built library). */
int bb_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* bb_status_str(int status);

/*
 * Build the per-head random-block table on the host.
 * Source: page "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
 * section "随机块掩码是如何生成的": one table per head, one row per middle block,
 * num_rand_blocks ids drawn from the middle blocks with the row's own window
 * removed.
 *
 *   seed      64-bit seed (the reference layer uses the layer index).
 *   H, L      heads and sequence length; block divides L; nb = L/block >= 3.
 *   r         random blocks per middle row; 0 <= r <= max(0, nb-5).
 *   rand_idx  HOST buffer of H*(nb-2)*r int32, caller-allocated, written as
 *             [H][nb-2][r]; row i-1 belongs to middle block i.
 * Each row is a uniform r-subset of {1..nb-2} \ {i-1, i, i+1}, stored in
 * ascending order.  Draws: SplitMix64 (Steele, Lea & Flood 2014), one stream
 * per head seeded from (seed, h); bounded integers by Lemire's (2019)
 * multiply-shift method with rejection; partial Fisher-Yates shuffle.  The
 * same arguments give the same bytes on every machine.
 * Errors: BB_ERR_SHAPE (sizes), BB_ERR_NULL (rand_idx NULL while H*(nb-2)*r > 0).
 */
int bb_rand_idx_build(uint64_t seed, int H, int L, int block, int r, int32_t* rand_idx);

/*
 * bb_rand_idx_build with the random range capped: the page's layer draws its
 * random blocks only from the first last_idx tokens (page "models 仓库中的 BigBird：
 * 线性复杂度稀疏注意力与长序列训练的完整实践", section "随机块掩码是如何生成的").
 * A block counts when it lies wholly before token last_idx: row i takes r
 * distinct ids from {1 .. min(nb-2, last_idx/block - 1)} \ {i-1, i, i+1}.
 *   last_idx  cap in tokens; <= 0, or >= (nb-1)*block: no cap (the same bytes
 *             as bb_rand_idx_build for the same arguments).
 * Same generator, order and output layout as bb_rand_idx_build.
 * Errors: as bb_rand_idx_build; BB_ERR_SHAPE also when some row keeps fewer
 * than r candidates under the cap (nothing is written then).
 */
int bb_rand_idx_build_capped(uint64_t seed, int H, int L, int block, int r, int last_idx,
                             int32_t* rand_idx);

/*
 * Validate a HOST random-block table [H][nb-2][r]: every entry in 1..nb-2,
 * outside {i-1, i, i+1} for its middle block i, no repeat within a row.  Row
 * order is free.  Returns BB_OK, BB_ERR_RAND_IDX, BB_ERR_SHAPE or BB_ERR_NULL.
 */
int bb_rand_idx_check(const int32_t* rand_idx, int H, int L, int block, int r);

/*
 * Bytes of device workspace bb_attn_forward needs for these sizes: the
 * split-K partial results (row max, row sum, unnormalised output, fp32) of
 * the two global query blocks of every (b, h), or, for problems small enough
 * to be split over their key tiles (BB_ORDINARY_UNITS), of every query block's
 * key chunks, for the largest r the sizes allow.  0 for empty inputs.  Returns
 * 0 also for unsupported sizes (bb_attn_forward then reports BB_ERR_SHAPE).
 */
size_t bb_attn_workspace_bytes(int B, int H, int L, int d, int block);

/*
 * How bb_attn_forward_ex with `flags` runs these sizes, without launching
 * anything: *n_units = work units of its unit launch(es) (64 query rows
 * against a list of key tiles each), *small = 1 when the problem is split
 * over the key tiles of every query block (see BB_ORDINARY_UNITS), else 0.
 * Same size, dtype and flag checks as the forward (no pointer checks);
 * outputs untouched on an error.  For tools and benchmarks that name the
 * kernels a call runs.
 */
int bb_attn_forward_plan(int B, int H, int L, int d, int block, int r, int dtype, unsigned flags,
                         long long* n_units, int* small);

/*
 * BigBird block-sparse self-attention forward.
 *
 *   q, k, v    DEVICE [B][H][L][d] in `dtype` (bf16 or fp32), 16-byte aligned.
 *   pad_mask   DEVICE uint8 [B][L], nonzero = real token, 0 = padding (the key
 *              gets -10000 added to its logit), 8-byte aligned; or NULL for
 *              no padding.  Only the key side is masked; padded query rows are
 *              computed by the same rule.
 *   rand_idx   DEVICE int32 [H][nb-2][r]; validate it with bb_rand_idx_check
 *              first (the kernels clamp entries into 1..nb-2 so a bad table
 *              cannot read out of bounds, but its result is then undefined).
 *              May be NULL when r == 0.
 *   B, H, L    batch, heads, sequence length (B == 0 or H == 0: no-op, BB_OK).
 *   d          head dimension; must be 64.
 *   block      block size; 64 or 128; L % block == 0; nb = L/block >= 3;
 *              L <= 64 * 65535 (64-key tile ids are 16-bit).
 *   r          random blocks per middle row, 0 <= r <= max(0, nb-5) (at nb-5 every
 *              middle row attends every block).
 *   out        DEVICE [B][H][L][d] in `dtype`, 16-byte aligned, fully
 *              overwritten; must not overlap q, k or v.
 *   dtype      BB_BF16 (fp32 accumulation, bf16 output rounded to nearest
 *              even) or BB_FP32.  q, k and v must be finite: the kernels are
 *              built without NaN semantics, so NaN or Inf inputs give
 *              unspecified (but memory-safe) outputs.
 *   workspace  DEVICE buffer of at least bb_attn_workspace_bytes(...) bytes,
 *              256-byte aligned.  Its contents need no initialisation (every
 *              byte read is written earlier in the same call).  Calls that run
 *              concurrently need distinct workspaces.
 *   stream     hipStream_t to enqueue on (NULL = the null stream).
 * The call is asynchronous: results are valid once `stream` has been
 * synchronised.  Launch errors map to BB_ERR_HIP.
 */
int bb_attn_forward(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                    const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                    void* out, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc -- the
 * forward of bb_attn_forward without a workspace argument: its split-K
 * partials go to a scratch area the library holds in each GPU's memory (a
 * file-scope device array of BB_NOALLOC_SCRATCH_BYTES, present from the
 * library's load until the process ends).  The call allocates and frees
 * nothing; the first call on a device looks the area's address up once
 * (hipGetSymbolAddress) and keeps it.
 *   Arguments as bb_attn_forward (the fused launch), without workspace.
 *   Errors as bb_attn_forward; BB_ERR_WORKSPACE when these sizes need more
 *   than BB_NOALLOC_SCRATCH_BYTES of partials (bb_attn_workspace_bytes()).
 * Every call on a GPU shares that GPU's area: calls that overlap on one GPU
 * (on other streams or from other threads) race and give undefined results;
 * order them on one stream.  Nothing needs clearing between calls (every
 * byte a call reads is written earlier in the same call).
 */
#define BB_NOALLOC_SCRATCH_BYTES (64u << 20)
int bb_attn_forward_noalloc(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                            const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                            void* out, int dtype, void* stream);

/* bb_attn_forward with flags: a launch mode (BB_LAUNCH_FUSED or BB_LAUNCH_SPLIT,
 * which give the same result bit for bit), optionally one phase
 * (BB_PHASE_UNITS or BB_PHASE_MERGE) for callers that time the phases or
 * enqueue other work between them, optionally BB_QUERY_MASK (the pair
 * masking variant) and BB_ORDINARY_UNITS.  Unknown flags: BB_ERR_SHAPE. */
int bb_attn_forward_ex(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                       const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                       void* out, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream, unsigned flags);

/* bb_attn_forward_ex that also timestamps its kernels: start_event and
 * stop_event (hipEvent_t created by the caller with timing enabled, or NULL)
 * are recorded by the launches themselves at the start of the first and the
 * end of the last kernel the call enqueues (with BB_PHASE_UNITS: exactly the
 * work-unit launch), so hipEventElapsedTime between them is the kernels'
 * execution time without enqueue gaps.  Same arguments, checks and errors as
 * bb_attn_forward_ex; events are not touched when the call returns an error
 * before launching. */
int bb_attn_forward_timed(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                          const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                          void* out, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream, unsigned flags, void* start_event, void* stop_event);

/*
 * bb_attn_forward that also writes the row log-sum-exp a backward pass needs.
 * Source: the softmax of page "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
 * section "BigBird：从二次方注意力到线性稀疏注意力"; the same page's encoder section
 * trains the layer with the forward recomputed in the backward pass.
 *   lse   DEVICE float [B][H][L], 4-byte aligned, caller-allocated: for every
 *         query row t, log(sum_u exp(s_tu)) (natural log) over its allowed keys,
 *         s_tu = q.k/sqrt(d) - 10000 [key u padded], the logits of the softmax.
 *         For bf16 the row sum is that of the bf16-rounded probabilities the
 *         output is formed from.  Must not be NULL when B*H > 0.
 * Everything else as bb_attn_forward (the fused launch).
 */
int bb_attn_forward_lse(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                        const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                        void* out, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream, float* lse);

/* bb_attn_forward_lse with flags: BB_QUERY_MASK (pair masking; then the
 * log-sum-exp of a padded query row leaves out the row's uniform -10000
 * offset -- it cancels in that row's softmax and in the backward's rebuilt P,
 * and kept, an fp32 value near -10000 would hold the row's log-sum-exp to
 * about 1e-3) and BB_ORDINARY_UNITS.  Other flags: BB_ERR_SHAPE. */
int bb_attn_forward_lse_ex(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                           const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                           void* out, int dtype, void* workspace, size_t workspace_bytes,
                           void* stream, float* lse, unsigned flags);

/*
 * Invert a HOST random-block table for the backward pass: for every head h
 * and key block j, the middle query blocks i (ascending) whose row
 * rand_idx[h][i-1][:] holds j.
 *   inv_off   HOST int32 [H][nb+1], caller-allocated: rows of (h, j) are
 *             inv_rows[inv_off[h][j] .. inv_off[h][j+1]) (absolute offsets).
 *   inv_rows  HOST int32 [H * (nb-2) * r], caller-allocated (may be NULL when r == 0).
 * The table is validated first (bb_rand_idx_check's errors).  Copy both
 * arrays to the device for bb_attn_backward.
 */
int bb_rand_idx_invert(const int32_t* rand_idx, int H, int L, int block, int r, int32_t* inv_off,
                       int32_t* inv_rows);

/* Bytes of device workspace bb_attn_backward needs (0 for empty or
 * unsupported sizes): the rows' (LSE, D) pairs and fp32 partials of dQ, dK
 * and dV -- of the global blocks' chunks, or for small problems (see
 * BB_ORDINARY_UNITS) of every block's chunks. */
size_t bb_attn_backward_workspace_bytes(int B, int H, int L, int d, int block);

/*
 * Backward pass of the same attention: the gradients of sum(out * dout)
 * with respect to q, k and v (the pad offset is a constant).  The gradient
 * of softmax attention restricted to the block pattern of bb_attn_forward:
 * P rebuilt from lse, D_t = dout_t . out_t, dS = P (dout V^T - D),
 * dq = dS K / sqrt(d), dk = dS^T Q / sqrt(d), dv = P^T dout.
 *   q, k, v, pad_mask, rand_idx, B, H, L, d, block, r
 *              as passed to the forward that produced out and lse.
 *   inv_off, inv_rows
 *              DEVICE copies of bb_rand_idx_invert's output for rand_idx
 *              (inv_rows may be NULL when r == 0).  Offsets are clamped
 *              into the table and entries into 1..nb-2, so a wrong table
 *              cannot read out of bounds (its result is then undefined).
 *   out, lse   DEVICE forward output [B][H][L][d] and bb_attn_forward_lse's lse.
 *   dout       DEVICE upstream gradient [B][H][L][d].
 *   dq, dk, dv DEVICE [B][H][L][d], fully overwritten; must not overlap each
 *              other or any input.
 *   dtype      BB_BF16 (fp32 accumulation, bf16 results rounded to nearest
 *              even) or BB_FP32, as the forward.
 *   block      64 or 128, as the forward.
 *   workspace  DEVICE, >= bb_attn_backward_workspace_bytes(), 256-byte aligned,
 *              no initialisation needed; concurrent calls need distinct ones.
 * Alignment: q, k, v, out, dout, dq, dk, dv 16 bytes; pad_mask 8; lse,
 * inv_off, inv_rows, rand_idx 4.  Asynchronous on `stream`, like the forward;
 * nothing is launched when a check fails.
 */
int bb_attn_backward(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                     const int32_t* rand_idx, const int32_t* inv_off, const int32_t* inv_rows,
                     int B, int H, int L, int d, int block, int r, const void* out, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* bb_attn_backward with flags: BB_QUERY_MASK, the gradients of the
 * pair-masked forward (out and lse from bb_attn_forward_lse_ex with the same
 * flag), and BB_ORDINARY_UNITS (no small-problem split).  Other flags:
 * BB_ERR_SHAPE. */
int bb_attn_backward_ex(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                        const int32_t* rand_idx, const int32_t* inv_off, const int32_t* inv_rows,
                        int B, int H, int L, int d, int block, int r, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream, unsigned flags);

/*
 * The attention layer around the op: input projections of the hidden states
 * to query, key and value (key_dim = hidden / heads), the block-sparse
 * attention of bb_attn_forward, and the output projection of the
 * concatenated heads.  Source: page "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的
 * 完整实践", the layer's construction (projections of width hidden / heads per
 * head) and section "BigBird：从二次方注意力到线性稀疏注意力" (the attention).
 *   [q | k | v] = x w_qkv^T + b_qkv, split into H heads of 64;
 *   o = attention(q, k, v) (bb_attn_forward's definition, the same pad_mask and
 *   rand_idx); y = concat_heads(o) w_o^T + b_o.
 *   x          DEVICE bf16 [B][L][hidden], 16-byte aligned.
 *   w_qkv      DEVICE bf16 [3*hidden][hidden] (rows: q outputs, then k, then v;
 *              the [out][in] layout of a linear layer), 16-byte aligned.
 *   b_qkv      DEVICE float [3*hidden], 16-byte aligned.
 *   w_o, b_o   DEVICE bf16 [hidden][hidden], float [hidden], 16-byte aligned.
 *   pad_mask, rand_idx, block, r
 *              as bb_attn_forward.
 *   hidden     H * 64, a multiple of 128; L a multiple of 128 and of block.
 *   y          DEVICE bf16 [B][L][hidden], fully overwritten, must not overlap x.
 *   dtype      BB_BF16 only (fp32 accumulation; q, k, v and the attention output
 *              are stored as bf16 between the steps).
 *   workspace  DEVICE, >= bb_layer_workspace_bytes(), 256-byte aligned.
 * Asynchronous on `stream`; checks as bb_attn_forward, nothing launched on error.
 */
size_t bb_layer_workspace_bytes(int B, int L, int hidden, int H, int block);
int bb_layer_forward(const void* x, const void* w_qkv, const float* b_qkv, const void* w_o, const float* b_o,
                     const uint8_t* pad_mask, const int32_t* rand_idx, int B, int L, int hidden, int H,
                     int block, int r, void* y, int dtype, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * A stack of n_layers attention layers (bb_layer_forward's layer), each
 * with its own weights and its own random-block table: the pages' encoder
 * stacks its layers and seeds each layer's table with the layer's index
 * (page "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
 * sections "随机块掩码是如何生成的" and "BigBirdEncoder 的关键参数").
 *   h_0 = x;  h_l = layer_l(h_{l-1}) for l = 1..n_layers;  y = h_{n_layers}.
 *   w_qkv, b_qkv, w_o, b_o, rand_idx
 *              HOST arrays of n_layers DEVICE pointers, entry l for layer l+1,
 *              each as bb_layer_forward takes it (rand_idx may be NULL when
 *              r == 0).  Build table l with bb_rand_idx_build(seed = l, ...)
 *              for the pages' convention.
 *   n_layers   >= 1.
 *   workspace  DEVICE, >= bb_layer_stack_workspace_bytes(): one layer's
 *              workspace and one activation buffer [B][L][hidden] bf16.
 *   y          must overlap neither x nor the workspace, which must not overlap
 *              x (BB_ERR_ALIAS).
 *   Everything else as bb_layer_forward (the same pad_mask for every layer).
 * Activations between layers are stored as bf16.  Every argument of every
 * layer is checked before the first launch; nothing is launched on an error.
 * Asynchronous on `stream`.
 */
size_t bb_layer_stack_workspace_bytes(int B, int L, int hidden, int H, int block);
int bb_layer_stack_forward(const void* x, const void* const* w_qkv, const float* const* b_qkv,
                           const void* const* w_o, const float* const* b_o, const uint8_t* pad_mask,
                           const int32_t* const* rand_idx, int n_layers, int B, int L, int hidden, int H,
                           int block, int r, void* y, int dtype, void* workspace, size_t workspace_bytes,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BB_ATTN_H_ */
