/*
 * ssd.h -- C ABI of libssd.so: the Mamba2 SSD chunked selective scan over
 * variable-length packed batches, for AMD Instinct MI355X (gfx950).
 *
 * The problem follows three public vLLM pull requests:
 *  - "[Model] Mamba2 varlen and metadata refactor" (PR #21467), Purpose:
 *    requests are packed along one token axis, (total_tokens, hidden), with
 *    cu_seqlens marking where each request starts, and the batch metadata is
 *    prepared once and shared by every layer;
 *  - "[Bugfix] Mamba2 SSD varlen bug fix initstates decay, improve test, assert
 *    chunk pwr 2" (PR #21783), Purpose: the initial or previous-chunk state
 *    must be scaled by the decay accumulated up to and including each token,
 *    chunk_size must be a power of two, and it does not change the result;
 *  - "[Model Runner V2] Automatic prefix caching for GDN hybrid models"
 *    (PR #54637), Purpose and the block-checkpoint scatter diff fragment:
 *    the chunk kernel exports per-chunk states, the state at each cache-block
 *    boundary is written to the slot the block table names, sequences whose
 *    computed prefix is not chunk-aligned get no interior checkpoints, and
 *    the block size must be a multiple of the kernel chunk size.
 *
 * What is computed (per sequence s, head h, group g = h / (nheads/ngroups)):
 *     delta_t = softplus(dt[t,h] + dt_bias[h])
 *     h_t     = exp(delta_t * A[h]) * h_{t-1} + delta_t * x_t (outer) B_t[g]
 *     y_t     = h_t . C_t[g] + D[h] * x_t
 * starting from initial_states[s,h] (if flagged) or zero; evaluated tile by
 * tile of min(chunk_size, 64) tokens (intra-tile quadratic form + state passing
 * between tiles, an exact re-association of the recurrence), with chunk_size
 * fixing the chunk grid and the exported states.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked [host]. Tensors are dense,
 *    row-major and contiguous. Layouts: x, y (T, H, P); dt (T, H);
 *    B, C (T, G, N); A, dt_bias, D (H); states (., H, P, N) float32.
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronise the host. Inputs must stay unchanged and
 *    outputs untouched until the stream has passed the call.
 *  - The caller allocates and owns every buffer; the library allocates and
 *    frees nothing, keeps no mutable global state, and is reentrant.
 *  - Argument errors (shape, size, NULL, unsupported configuration) are
 *    returned synchronously before anything is launched.
 *  - Data errors only visible on the device (malformed cu_seqlens, more chunks
 *    than max_chunks, a cache slot out of range, a touched block beyond the
 *    block table) are OR-ed into the sticky device word `error_flag` as the
 *    SSD_DATA_* bits below; the affected work is skipped, never read or
 *    written out of bounds. The caller clears the flag and reads it back.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
    SSD_ERR_CHUNK_SIZE = 2,   /* chunk_size not a power of two in [16, 256] */
    SSD_ERR_SHAPE = 3,        /* negative/zero sizes, nheads % ngroups != 0, ... */
    SSD_ERR_BLOCK_SIZE = 4,   /* block_size <= 0 or not a multiple of chunk_size */
    SSD_ERR_CAPACITY = 5,     /* max_chunks < total_tokens/chunk_size + nseqs, or a too small output capacity */
    SSD_ERR_DTYPE = 6,        /* unknown ssd_dtype */
    SSD_ERR_HIP = 7,          /* a HIP launch or attribute call failed */
    SSD_ERR_UNSUPPORTED = 8   /* headdim not a multiple of 16, or dstate not supported for the dtype */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Bits of the sticky device error word. */
#define SSD_DATA_BAD_CU_SEQLENS 1   /* cu_seqlens[0] != 0, decreasing, or last != total_tokens */
#define SSD_DATA_TOO_MANY_CHUNKS 2  /* sum of ceil(len/chunk_size) > max_chunks */
#define SSD_DATA_BAD_SLOT 4         /* a cache slot >= its buffer's slot count */
#define SSD_DATA_BAD_BLOCK 8        /* a touched block index >= max_blocks_per_seq */

/*
 * Varlen chunk metadata of one packed batch (built once, shared by all layers).
 * The struct itself lives in host memory; its array fields are device buffers
 * the caller owns. Chunk k of sequence s covers tokens
 *     [cu_seqlens[s] + k*chunk_size, min(cu_seqlens[s] + (k+1)*chunk_size, cu_seqlens[s+1]))
 * i.e. the chunk grid restarts at every sequence start and no chunk spans two
 * sequences; chunks are numbered in packed order.
 */
typedef struct {
    int32_t nseqs;             /* [host] number of sequences S >= 0 */
    int32_t total_tokens;      /* [host] T = cu_seqlens[S] */
    int32_t chunk_size;        /* [host] power of two in [16, 256] */
    int32_t max_chunks;        /* [host] capacity, >= T/chunk_size + S (an upper bound of the chunk count) */
    const int32_t *cu_seqlens; /* in  [S+1] prefix sums of the sequence lengths */
    int32_t *chunk_offsets;    /* out [max_chunks+1] first token of each chunk; T past the last chunk */
    int32_t *chunk_seq_idx;    /* out [max_chunks] sequence of each chunk; -1 past the last chunk */
    int32_t *seq_chunk_start;  /* out [S+1] first chunk of each sequence; [S] = number of chunks */
    int32_t *nchunks;          /* out [1] number of chunks */
    int32_t *seq_order;        /* out [S] sequences by decreasing length, ties by index (work order) */
    int32_t *error_flag;       /* in/out [1] sticky SSD_DATA_* bits */
} ssd_varlen_meta;

/*
 * Builds the chunk metadata from cu_seqlens (varlen layout: "Mamba2 varlen and
 * metadata refactor", Purpose). One small launch; bit-exact integer output.
 * Errors: SSD_ERR_NULL_ARG (meta or any buffer NULL; seq_order may not be
 * NULL), SSD_ERR_SHAPE (nseqs < 0, total_tokens < 0), SSD_ERR_CHUNK_SIZE,
 * SSD_ERR_CAPACITY (max_chunks below the bound), SSD_ERR_HIP.
 * Device data errors: SSD_DATA_BAD_CU_SEQLENS (outputs then undefined).
 */
ssd_status ssd_varlen_metadata(const ssd_varlen_meta *meta, void *stream);

/*
 * The chunked scan over the varlen layout of "[Model] Mamba2 varlen and
 * metadata refactor" (Purpose: packed (total_tokens, hidden) inputs, one
 * cu_seqlens, per-sequence initial states), with the decay indexing of
 * "[Bugfix] Mamba2 SSD varlen bug fix initstates decay, improve test, assert
 * chunk pwr 2" (Purpose: the entering state reaches token i through the
 * inclusive cumsum at i, and the chunk's total decay is read at its last valid
 * token; chunk_size a power of two) and the per-chunk state export of
 * "[Model Runner V2] Automatic prefix caching for GDN hybrid models" (Purpose,
 * kernels/layers item). For every
 * chunk, delta = softplus(dt + dt_bias) and the chunk-local inclusive cumsum of
 * delta*A; C.B^T with the segment-sum decay mask; the intra-chunk output
 * (L o CB) . (delta x); the inter-chunk output exp(cumsum_i) * C_i . h_in; the
 * chunk's own state, and the state passed to the next chunk
 * h_out = exp(cumsum_last) * h_in + sum_j exp(cumsum_last - cumsum_j) delta_j x_j B_j^T.
 * The first chunk of a sequence starts from initial_states[s] when
 * has_initial_state[s] != 0 (all, if has_initial_state is NULL), else from 0.
 *
 *  x, B, C, y      element type `in_dtype` (SSD_F32 or SSD_BF16); y gets x's type
 *  dt              float32 (T, H), raw (before bias and softplus)
 *  dt_bias, D      float32 (H) or NULL (= 0)
 *  A               float32 (H), per-head log-decay rate (normally negative)
 *  initial_states  float32 (S, H, P, N) or NULL (all start from zero)
 *  final_states    float32 (S, H, P, N), written for every sequence
 *  chunk_states    optional float32 state export (the per-chunk export of the
 *                  prefix-caching page): the state AFTER the last token of a
 *                  chunk. With chunk_state_dst == NULL, chunk c's state goes to
 *                  chunk_states[c] (capacity >= meta->max_chunks). With
 *                  chunk_state_dst != NULL (e.g. the plan of
 *                  ssd_export_chunk_states), it goes to
 *                  chunk_states[chunk_state_dst[c]] when that is >= 0, so a
 *                  block-aligned checkpoint is written straight into a state
 *                  cache of `chunk_states_capacity` slots; slots >= capacity
 *                  raise SSD_DATA_BAD_SLOT and are skipped.
 * Supported: headdim a multiple of 16; dstate in {16, 32, 64, 128, 256} for
 * bf16 and {16, 32, 64, 128} for f32; nheads % ngroups == 0.
 * Precision: all decay, state and accumulation arithmetic is float32. For
 * bf16 inputs the matrix-core operands derived in float32 (the masked decay
 * matrix, delta-scaled x, and the carried state) are rounded to bf16.
 * Errors: SSD_ERR_NULL_ARG, SSD_ERR_SHAPE, SSD_ERR_DTYPE, SSD_ERR_UNSUPPORTED,
 * SSD_ERR_CAPACITY (chunk_states_capacity < max_chunks with no dst map, or <= 0),
 * SSD_ERR_HIP. If error_flag already holds SSD_DATA_BAD_CU_SEQLENS the kernel
 * writes nothing.
 * There is no workspace argument (and no workspace-size query): the scan is
 * one fused walk per (sequence, head, headdim tile) that keeps the chunk
 * cumsums, the C.B^T tiles and the carried state in LDS and registers, so no
 * intermediate is materialised in device memory.
 */
ssd_status ssd_chunk_scan_varlen(
    const void *x, const float *dt, const float *dt_bias, const float *A, const void *B,
    const void *C, const float *D, ssd_dtype in_dtype, const ssd_varlen_meta *meta,
    int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
    const float *initial_states, const int32_t *has_initial_state, void *y,
    float *final_states, float *chunk_states, const int32_t *chunk_state_dst,
    int32_t chunk_states_capacity, void *stream);

/*
 * Block-aligned checkpoint plan and scatter (the block-checkpoint scatter of
 * the prefix-caching page). Sequence s was computed up to absolute position
 * ncomp = num_computed_tokens[s] (NULL = 0) and this batch schedules its
 * L_s tokens, positions [ncomp, ncomp + L_s). The blocks of block_size tokens
 * touched are first = ncomp/block_size .. last = (ncomp + L_s - 1)/block_size.
 *  - Interior blocks k in [first, last) get the state after the chunk that
 *    ends at the block's end, chunk seq_chunk_start[s] + ((k+1)*block_size -
 *    ncomp)/chunk_size - 1 (clamped to the sequence's own chunks), and only
 *    when ncomp % chunk_size == 0 (otherwise no chunk ends there exactly and
 *    nothing is written for them).
 *  - Block `last` gets the sequence's final state (its last chunk's state).
 * Outputs (always written):
 *  ckpt_src         [nseqs * max_blocks_per_seq] source chunk of each block, or -1
 *  chunk_state_dst  [meta->max_chunks] slot block_table[s][k] that chunk c's
 *                   state goes to, or -1 (pass it to ssd_chunk_scan_varlen to
 *                   write checkpoints at the source)
 * If chunk_states != NULL (a dense per-chunk export [max_chunks, state_elems]
 * from the scan), the states are also copied now:
 *     state_cache[block_table[s][k]] = chunk_states[ckpt_src[s][k]].
 * block_table: int32 [nseqs, max_blocks_per_seq]; negative entries = no slot.
 * state_elems = nheads*headdim*dstate floats per state; num_slots = slots in
 * state_cache. Slot ids must be unique (duplicates: unspecified winner).
 * Errors: SSD_ERR_NULL_ARG, SSD_ERR_SHAPE, SSD_ERR_BLOCK_SIZE
 * (block_size <= 0 or % chunk_size != 0), SSD_ERR_HIP. Device data errors:
 * SSD_DATA_BAD_BLOCK, SSD_DATA_BAD_SLOT (those entries are skipped).
 */
ssd_status ssd_export_chunk_states(
    const ssd_varlen_meta *meta, const int32_t *num_computed_tokens, const int32_t *block_table,
    int32_t max_blocks_per_seq, int32_t block_size, int32_t *ckpt_src, int32_t *chunk_state_dst,
    const float *chunk_states, int32_t state_elems, float *state_cache, int32_t num_slots,
    void *stream);

/*
 * One decode step with dual state anchors (the decode kernels' read/write
 * anchor split on the prefix-caching page: a step reads the running state from
 * the previous step's anchor slot and writes to the current one, so a cached
 * block checkpoint is never overwritten in place). One new token per sequence:
 *     S     = state_cache[read_slot[s], h]     (zero when read_slot[s] < 0)
 *     delta = softplus(dt[s,h] + dt_bias[h])
 *     S'    = exp(delta * A[h]) * S + delta * x[s,h] (outer) B[s,g]
 *     y[s,h] = S' . C[s,g] + D[h] * x[s,h]
 *     state_cache[write_slot[s], h] = S'       (skipped when write_slot[s] < 0)
 * with g = h / (nheads / ngroups): the same recurrence as the scan, one token.
 *
 *  x, B, C, y      element type `in_dtype`; x, y (nseqs, H, P); B, C (nseqs, G, N)
 *  dt              float32 (nseqs, H), raw; dt_bias, D float32 (H) or NULL (= 0)
 *  A               float32 (H)
 *  state_cache     float32 (num_slots, H, P, N), 16-byte aligned, updated in place
 *  read_slot,      int32 (nseqs) device arrays. read_slot[s] == write_slot[s]
 *  write_slot      is an in-place update. Write slots must be unique and must
 *                  not be another sequence's read slot (else unspecified).
 *  error_flag      int32 [1] device sticky flag, or NULL. A slot >= num_slots
 *                  sets SSD_DATA_BAD_SLOT; that sequence is skipped entirely
 *                  (no y, no state written).
 * Supported: dstate in {16, 32, 64, 128, 256}, any headdim >= 1.
 * Precision: float32 state and arithmetic (hardware exp2/log2); y rounded to
 * x's type (round to nearest even for bf16).
 * Errors (returned before any launch): SSD_ERR_DTYPE, SSD_ERR_SHAPE (sizes,
 * nheads % ngroups, unaligned state_cache), SSD_ERR_UNSUPPORTED (dstate),
 * SSD_ERR_NULL_ARG; SSD_ERR_HIP on a failed launch. Asynchronous on `stream`;
 * the caller owns every buffer.
 */
ssd_status ssd_decode_step(
    const void *x, const float *dt, const float *dt_bias, const float *A, const void *B,
    const void *C, const float *D, ssd_dtype in_dtype, int32_t nseqs, int32_t nheads,
    int32_t headdim, int32_t dstate, int32_t ngroups, float *state_cache, int32_t num_slots,
    const int32_t *read_slot, const int32_t *write_slot, void *y, int32_t *error_flag,
    void *stream);

/*
 * Continuation: how many tokens the scheduler gives each prefilling sequence
 * this step (the scheduler diff fragment of the prefix-caching page, "re-align
 * a misaligned start at the next boundary, otherwise clip the end down", with
 * the review note under it: re-align a misaligned start even on the final
 * bite, and let the final bite from an aligned start end anywhere). HOST code:
 * every pointer is a [host] array of nseqs entries; nothing is launched.
 * For sequence s with start = num_computed_tokens[s] tokens already computed
 * (e.g. a prefix whose state was loaded from the cache), prompt_len[s] tokens
 * in all and a budget of budget[s] tokens this step:
 *     last_aligned = floor(prompt_len / align) * align
 *     end = min(start + budget, prompt_len)
 *     if start % align != 0 and the next multiple of align is <= last_aligned:
 *         end = min(end, that multiple)            (re-align)
 *     else if end < last_aligned:
 *         end = floor(end / align) * align         (clip down)
 *     num_scheduled[s] = end - start
 * With align the cache block size (a multiple of chunk_size), every bite after
 * a misaligned first one starts on a block boundary, so the chunk grid of each
 * bite (anchored at its first token) falls on absolute multiples of
 * chunk_size and every block end inside the bite is a chunk end: the plan of
 * ssd_export_chunk_states (called with num_computed_tokens = the bite starts)
 * then writes an exact checkpoint for every block that ends in the computed
 * range; the misaligned first bite ends at a block end, whose checkpoint is
 * its final state.
 * Errors: SSD_ERR_NULL_ARG (a NULL array with nseqs > 0), SSD_ERR_SHAPE
 * (nseqs < 0, align <= 0, a budget below align, a start outside
 * [0, prompt_len]); num_scheduled is left unspecified on error.
 */
ssd_status ssd_prefill_bites(int32_t nseqs, const int32_t *num_computed_tokens, const int32_t *prompt_len,
                             const int32_t *budget, int32_t align, int32_t *num_scheduled);

/*
 * Chunked gated delta rule with per-chunk state export: the recurrent state of
 * the GDN layers of the prefix-caching page (Purpose, kernels/layers item:
 * "per-chunk intermediate-state export from the FLA chunk kernel"; chunk size
 * 64 in its per-file table). The pages print no formula; the gated delta rule
 * read here is, per sequence s and value head h (key head g = h / (H/G)), with
 * the state S (dv x dk) value-major:
 *     S_t = e^(gate[t,h]) S_{t-1} (I - beta[t,h] k_t k_t^T) + beta[t,h] v_t k_t^T
 *     o_t = scale S_t q_t
 * from initial_states[s,h] (if flagged; all if has_initial_state is NULL) or
 * zero, evaluated 64 tokens at a time in the chunked (WY) form.
 *  q, k            bf16 (T, G, dk); the layer normalises them before the call
 *  v, o            bf16 (T, H, dv)
 *  gate, beta      float32 (T, H): log-decay (<= 0) and write strength
 *  initial_states  float32 (S, H, dv, dk) or NULL; final_states (S, H, dv, dk)
 *  chunk_states    optional state export after each chunk, as for the scan:
 *                  chunk_states[chunk_state_dst[c]] (or [c] when
 *                  chunk_state_dst is NULL); slots >= capacity raise
 *                  SSD_DATA_BAD_SLOT and are skipped.
 * meta is the chunk metadata of ssd_varlen_metadata with chunk_size 64; the
 * block-checkpoint plan of ssd_export_chunk_states (state_elems = H dv dk)
 * feeds chunk_state_dst. Supported: in_dtype SSD_BF16, dk 128, dv a multiple
 * of 64, nheads % nkheads == 0.
 * workspace: device memory of at least
 * ssd_gated_delta_workspace_size(meta->max_chunks, nheads) bytes, 16-byte
 * aligned, owned by the caller; it holds (I + A)^-1 of every chunk and head
 * between the call's two kernels and is free again when the call's work on
 * `stream` has finished. Calls that overlap in time need separate workspaces.
 * Errors: SSD_ERR_NULL_ARG, SSD_ERR_SHAPE, SSD_ERR_DTYPE, SSD_ERR_UNSUPPORTED
 * (another dtype, dk, dv or chunk size), SSD_ERR_CAPACITY (chunk_states or
 * workspace too small), SSD_ERR_HIP.
 * Asynchronous on `stream`; the caller owns every buffer.
 */
ssd_status ssd_gated_delta_chunk_varlen(
    const void *q, const void *k, const void *v, const float *gate, const float *beta, float scale,
    ssd_dtype in_dtype, const ssd_varlen_meta *meta, int32_t nheads, int32_t nkheads, int32_t dk, int32_t dv,
    const float *initial_states, const int32_t *has_initial_state, void *o, float *final_states,
    float *chunk_states, const int32_t *chunk_state_dst, int32_t chunk_states_capacity,
    void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes ssd_gated_delta_chunk_varlen needs for a batch whose
 * metadata has `max_chunks` and for `nheads` value heads (0 for no chunks). */
size_t ssd_gated_delta_workspace_size(int32_t max_chunks, int32_t nheads);

/*
 * ssd_gated_delta_chunk_varlen without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): it calls no hipMalloc, hipFree or
 * allocating routine and uses a static 32 MiB device array of the library
 * instead (one per GPU, held until the process ends). Same arguments, layouts
 * and results as ssd_gated_delta_chunk_varlen.
 * Limit: ssd_gated_delta_workspace_size(meta->max_chunks, nheads) <= 32 MiB
 * (max_chunks * nheads <= 4096), else SSD_ERR_CAPACITY before any work.
 * Every call on one GPU shares that array: calls that overlap in time on one
 * GPU (other streams, other threads) race and must not be issued. Nothing in
 * it needs clearing between calls. The first call on a device resolves the
 * array's address (hipGetSymbolAddress); SSD_ERR_HIP if that fails.
 */
ssd_status ssd_gated_delta_chunk_varlen_noalloc(
    const void *q, const void *k, const void *v, const float *gate, const float *beta, float scale,
    ssd_dtype in_dtype, const ssd_varlen_meta *meta, int32_t nheads, int32_t nkheads, int32_t dk, int32_t dv,
    const float *initial_states, const int32_t *has_initial_state, void *o, float *final_states,
    float *chunk_states, const int32_t *chunk_state_dst, int32_t chunk_states_capacity, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *ssd_status_string(ssd_status status);

/*
 * Varlen causal conv1d with a conv-state cache: the depthwise causal
 * convolution that produces the scan's inputs (the causal_conv1d kernel named
 * on the prefix-caching page, whose conv metadata that page builds together
 * with the rest of the batch metadata; here the kernel walks the chunk grid of
 * `meta`, filled by ssd_varlen_metadata on the same stream). The pages name the
 * kernel without its formula; this is the standard Mamba2 depthwise causal
 * convolution. For sequence s (tokens cu[s] .. cu[s+1]-1, L of them), token j
 * and channel c, with W = width:
 *     u_j = x[cu[s]+j, c]                               (j >= 0)
 *     u_j = conv_states[read_slot[s], W-1+j, c]         (-(W-1) <= j < 0; zero when read_slot[s] < 0)
 *     out[cu[s]+j, c] = act(bias[c] + sum_k weight[c,k] * u_{j-(W-1)+k})
 *     conv_states[write_slot[s], i, c] = u_{L-(W-1)+i}  (i = 0..W-2; skipped when write_slot[s] < 0)
 * act: activation 0 = identity, 1 = SiLU z / (1 + e^-z). Arithmetic in fp32
 * (fmaf over the taps in order, bias first), output rounded to nearest even.
 *
 *  x, out        element type `in_dtype`, (T, channels) row-major, 16-byte aligned
 *  weight        float32 (channels, width); bias float32 (channels) or NULL (= 0)
 *  conv_states   element type `in_dtype`, (num_slots, width-1, channels), 16-byte
 *                aligned; the last W-1 inputs of a sequence, oldest first
 *  read_slot, write_slot  int32 (nseqs) or NULL (= all -1): dual anchors
 *  channels      multiple of 8; width 1..4
 * Preconditions: write slots are distinct, and none is another sequence's read
 * slot; a sequence may read and write the same slot only if it spans at most
 * one chunk (its reads and its write are then made by the same lanes).
 * Empty sequences copy their read state (or zeros) to their write slot.
 * Errors: SSD_ERR_NULL_ARG, SSD_ERR_SHAPE (channels <= 0, num_slots < 0,
 * misaligned buffers), SSD_ERR_UNSUPPORTED (channels % 8, width outside 1..4,
 * unknown activation), SSD_ERR_DTYPE, SSD_ERR_CHUNK_SIZE / SSD_ERR_CAPACITY
 * (meta), SSD_ERR_HIP. Device data error: SSD_DATA_BAD_SLOT in
 * meta->error_flag (a slot >= num_slots, or read_slot == write_slot >= 0 for a
 * sequence of more than one chunk; that sequence is skipped: nothing of it
 * read or written).
 */
ssd_status ssd_causal_conv1d_varlen(
    const void *x, const float *weight, const float *bias, ssd_dtype in_dtype,
    const ssd_varlen_meta *meta, int32_t channels, int32_t width, int32_t activation,
    void *conv_states, int32_t num_slots, const int32_t *read_slot, const int32_t *write_slot,
    void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
