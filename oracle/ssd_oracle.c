/*
 * ssd_oracle.c -- plain, slow, obviously correct CPU reference for the Mamba2
 * SSD varlen scan, in float64.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header, table or helper with the HIP library.
 *
 * Sources (the pages are three public vLLM pull requests):
 *  - "[Model] Mamba2 varlen and metadata refactor" (vLLM PR #21467), Purpose:
 *    tokens of all requests are packed along one axis, (seqlen, hiddendim),
 *    with cu_seqlens marking where each request starts; metadata is built once.
 *  - "[Bugfix] Mamba2 SSD varlen bug fix initstates decay, improve test, assert
 *    chunk pwr 2" (vLLM PR #21783), Purpose: the initial (or previous-chunk)
 *    state must carry exactly the decay accumulated up to and including the
 *    current token; chunk_size must be a power of two and does not change the
 *    result.
 *  - "[Model Runner V2] Automatic prefix caching for GDN hybrid models"
 *    (vLLM PR #54637), Purpose and the diff fragment of the block-checkpoint
 *    scatter: per-chunk states are exported, and the state at each cache-block
 *    boundary is written to block_table slots; sequences whose computed prefix
 *    is not chunk-aligned get no interior checkpoints; the source chunk is
 *    clamped to the sequence's own chunks.
 *
 * The recurrence itself (the pages print no formula; this is the plainest
 * reading of the problem statement, with ZOH decay and Euler input):
 *     delta_t = softplus(dt[t,h] + dt_bias[h])
 *     h_t     = exp(delta_t * A[h]) * h_{t-1} + delta_t * x_t (outer) B_t
 *     y_t     = h_t . C_t + D[h] * x_t
 * run token by token per (sequence, head) from the sequence's initial state
 * (or zero). The chunked scan is an exact re-association of this map, so the
 * oracle does not chunk: chunk_size only decides where states are recorded.
 *
 * Layouts (row-major): x, y (T,H,P); dt (T,H); B, C (T,G,N); states (.,H,P,N).
 * Head h reads group g = h / (H/G).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Softplus, identity above 20 (the usual threshold; never reached by the
 * workloads' dt distribution). */
static double oracle_softplus(double u)
{
    if (u > 20.0)
        return u;
    return log1p(exp(u));
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * The recurrence oracle.
 *   chunk_size > 0 and chunk_states != NULL: after the last token of every
 *   chunk (chunks cut per sequence from its first token, chunk_size tokens
 *   each, the last one possibly shorter) the state is copied to
 *   chunk_states[c], c = the chunk's index in the packed batch.
 *   has_init == NULL with init != NULL means every sequence has one;
 *   init == NULL means all start from zero. dt_bias / D may be NULL (zero).
 * Returns 0, or -1 on bad shapes.
 */
int oracle_ssd_varlen(int32_t nseqs, const int32_t *cu_seqlens, int32_t nheads, int32_t headdim,
                      int32_t dstate, int32_t ngroups, const double *x, const double *dt,
                      const double *dt_bias, const double *A, const double *B, const double *C,
                      const double *D, const double *init, const int32_t *has_init,
                      int32_t chunk_size, double *chunk_states, double *y, double *final_states,
                      int32_t nthreads)
{
    const int64_t H = nheads, P = headdim, N = dstate, G = ngroups;
    if (nseqs < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0)
        return -1;
    const int64_t heads_per_group = H / G;

    /* index of each sequence's first chunk (only used to place chunk states) */
    int64_t *first_chunk = (int64_t *)calloc((size_t)nseqs + 1, sizeof(int64_t));
    if (!first_chunk)
        return -1;
    for (int32_t s = 0; s < nseqs; ++s) {
        int64_t len = (int64_t)cu_seqlens[s + 1] - cu_seqlens[s];
        int64_t nch = chunk_size > 0 ? (len + chunk_size - 1) / chunk_size : 0;
        first_chunk[s + 1] = first_chunk[s] + nch;
    }

    const int64_t npairs = (int64_t)nseqs * H;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t pair = 0; pair < npairs; ++pair) {
        const int64_t s = pair / H, h = pair % H;
        const int64_t g = h / heads_per_group;
        double *S = (double *)malloc((size_t)(P * N) * sizeof(double));
        if (!S)
            continue;
        const int start_from_init = init != NULL && (has_init == NULL || has_init[s] != 0);
        for (int64_t i = 0; i < P * N; ++i)
            S[i] = start_from_init ? init[((s * H + h) * P) * N + i] : 0.0;

        const int64_t t0 = cu_seqlens[s], t1 = cu_seqlens[s + 1];
        for (int64_t t = t0; t < t1; ++t) {
            const double u = dt[t * H + h] + (dt_bias ? dt_bias[h] : 0.0);
            const double delta = oracle_softplus(u);
            const double decay = exp(delta * A[h]);
            const double *xt = x + (t * H + h) * P;
            const double *Bt = B + (t * G + g) * N;
            const double *Ct = C + (t * G + g) * N;
            /* state update: h_t = decay * h_{t-1} + delta * x_t (outer) B_t */
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n)
                    S[p * N + n] = decay * S[p * N + n] + delta * xt[p] * Bt[n];
            /* output: y_t = h_t . C_t + D * x_t (the state already holds token t) */
            double *yt = y + (t * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += Ct[n] * S[p * N + n];
                yt[p] = acc + (D ? D[h] : 0.0) * xt[p];
            }
            /* record the state after the last token of each chunk */
            if (chunk_size > 0 && chunk_states != NULL) {
                const int64_t local = t - t0;
                if ((local + 1) % chunk_size == 0 || t == t1 - 1) {
                    const int64_t c = first_chunk[s] + local / chunk_size;
                    memcpy(chunk_states + ((c * H + h) * P) * N, S, (size_t)(P * N) * sizeof(double));
                }
            }
        }
        memcpy(final_states + ((s * H + h) * P) * N, S, (size_t)(P * N) * sizeof(double));
        free(S);
    }
    free(first_chunk);
    return 0;
}

/*
 * Chunk metadata by plain enumeration. Chunk k of sequence s covers tokens
 * [cu[s] + k*cs, min(cu[s] + (k+1)*cs, cu[s+1])); chunks never span sequences.
 * Entries past the last chunk hold total_tokens (offsets) and -1 (seq index).
 * seq_order lists sequences by decreasing length, ties by index.
 * Returns 0, -1 on malformed cu_seqlens, -2 when max_chunks is too small.
 */
int oracle_varlen_metadata(int32_t nseqs, const int32_t *cu_seqlens, int32_t chunk_size,
                           int32_t max_chunks, int32_t *chunk_offsets, int32_t *chunk_seq_idx,
                           int32_t *seq_chunk_start, int32_t *nchunks, int32_t *seq_order)
{
    if (cu_seqlens[0] != 0)
        return -1;
    for (int32_t s = 0; s < nseqs; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s])
            return -1;
    const int32_t T = cu_seqlens[nseqs];
    int32_t c = 0;
    for (int32_t s = 0; s < nseqs; ++s) {
        seq_chunk_start[s] = c;
        for (int32_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; t += chunk_size) {
            if (c >= max_chunks)
                return -2;
            chunk_offsets[c] = t;
            chunk_seq_idx[c] = s;
            ++c;
        }
    }
    seq_chunk_start[nseqs] = c;
    *nchunks = c;
    for (int32_t k = c; k <= max_chunks; ++k)
        chunk_offsets[k] = T;
    for (int32_t k = c; k < max_chunks; ++k)
        chunk_seq_idx[k] = -1;
    /* insertion sort by (length desc, index asc) */
    for (int32_t s = 0; s < nseqs; ++s)
        seq_order[s] = s;
    for (int32_t i = 1; i < nseqs; ++i) {
        int32_t v = seq_order[i], j = i - 1;
        int32_t lv = cu_seqlens[v + 1] - cu_seqlens[v];
        while (j >= 0) {
            int32_t u = seq_order[j];
            int32_t lu = cu_seqlens[u + 1] - cu_seqlens[u];
            if (lu > lv || (lu == lv && u < v))
                break;
            seq_order[j + 1] = u;
            --j;
        }
        seq_order[j + 1] = v;
    }
    return 0;
}

/*
 * Block-checkpoint plan, following the scatter loop of the prefix-caching page:
 * sequence s was computed up to absolute position ncomp (num_computed_tokens,
 * NULL = 0) and schedules L tokens, i.e. absolute positions [ncomp, ncomp+L).
 * Blocks first = ncomp / bs .. last = (ncomp + L - 1) / bs are touched.
 *  - interior blocks k in [first, last): only when ncomp % cs == 0; their
 *    state is the one after the chunk that ends at the block end, i.e. chunk
 *    first_chunk[s] + ((k+1)*bs - ncomp)/cs - 1, clamped into the sequence's
 *    own chunk range;
 *  - block `last`: the sequence's final state (= its last chunk's state).
 * ckpt_src[s*max_blocks + k] = that chunk index or -1. chunk_state_dst[c] is
 * the cache slot block_table[s*max_blocks + k] the chunk's state goes to, or
 * -1 (no block, or a negative slot).
 * Returns 0, or -3 when a touched block lies beyond max_blocks.
 */
int oracle_checkpoint_plan(int32_t nseqs, const int32_t *cu_seqlens, const int32_t *seq_chunk_start,
                           int32_t max_chunks, const int32_t *num_computed_tokens,
                           const int32_t *block_table, int32_t max_blocks, int32_t block_size,
                           int32_t chunk_size, int32_t *ckpt_src, int32_t *chunk_state_dst)
{
    for (int64_t i = 0; i < (int64_t)nseqs * max_blocks; ++i)
        ckpt_src[i] = -1;
    for (int32_t c = 0; c < max_chunks; ++c)
        chunk_state_dst[c] = -1;
    for (int32_t s = 0; s < nseqs; ++s) {
        const int64_t L = (int64_t)cu_seqlens[s + 1] - cu_seqlens[s];
        if (L <= 0)
            continue;
        const int64_t ncomp = num_computed_tokens ? num_computed_tokens[s] : 0;
        const int64_t first = ncomp / block_size, last = (ncomp + L - 1) / block_size;
        if (last >= max_blocks)
            return -3;
        const int64_t lo = seq_chunk_start[s], hi = seq_chunk_start[s + 1] - 1;
        if (ncomp % chunk_size == 0) {
            for (int64_t k = first; k < last; ++k) {
                int64_t src = lo + ((k + 1) * block_size - ncomp) / chunk_size - 1;
                if (src < lo)
                    src = lo;
                if (src > hi)
                    src = hi;
                ckpt_src[s * max_blocks + k] = (int32_t)src;
            }
        }
        ckpt_src[s * max_blocks + last] = (int32_t)hi;
        for (int64_t k = first; k <= last; ++k) {
            const int32_t src = ckpt_src[s * max_blocks + k];
            const int32_t slot = block_table[s * max_blocks + k];
            if (src >= 0 && slot >= 0)
                chunk_state_dst[src] = slot;
        }
    }
    return 0;
}

/*
 * Gated delta rule (the recurrent state of the GDN layers whose chunk kernel
 * the prefix-caching page extends with a per-chunk intermediate-state export,
 * chunk size 64). The pages print no formula; this is the plainest reading of
 * the gated delta rule, token by token, per sequence s and value head h (key
 * head g = h / (H/G)), with the state S (dv x dk, value-major):
 *     S      <- exp(gate[t,h]) * S                   (gated decay; gate <= 0)
 *     u      =  beta[t,h] * (v[t,h] - S k[t,g])       (delta-rule write value)
 *     S      <- S + u (outer) k[t,g]
 *     o[t,h] =  scale * S q[t,g]
 * i.e. S_t = e^(gate) S_{t-1} (I - beta k k^T) + beta v k^T, o_t = scale S_t q_t,
 * starting from initial_states[s,h] (if flagged) or zero. States are recorded
 * after the last token of each chunk (chunk grid per sequence from its first
 * token, like the scan's) when chunk_states is given, and after the last token
 * of the sequence in final_states. Layouts (row-major): q, k (T,G,dk);
 * v, o (T,H,dv); gate, beta (T,H); states (.,H,dv,dk).
 * OpenMP over (sequence, head) pairs. Returns 0, or -1 on bad shapes.
 */
int oracle_gated_delta(int32_t nseqs, const int32_t *cu_seqlens, int32_t H, int32_t G, int32_t dk,
                       int32_t dv, const double *q, const double *k, const double *v, const double *gate,
                       const double *beta, double scale, const double *init, const int32_t *has_init,
                       int32_t chunk_size, double *o, double *final_states, double *chunk_states)
{
    if (nseqs < 0 || H <= 0 || G <= 0 || H % G != 0 || dk <= 0 || dv <= 0)
        return -1;
    const int64_t per_state = (int64_t)dk * dv;
    int64_t *chunk_base = (int64_t *)calloc((size_t)nseqs + 1, sizeof(int64_t));
    if (!chunk_base)
        return -1;
    for (int32_t s = 0; s < nseqs; ++s) {
        const int64_t L = (int64_t)cu_seqlens[s + 1] - cu_seqlens[s];
        chunk_base[s + 1] = chunk_base[s] + (chunk_size > 0 ? (L + chunk_size - 1) / chunk_size : 0);
    }
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int32_t s = 0; s < nseqs; ++s) {
        for (int32_t hd = 0; hd < H; ++hd) {
            const int64_t g = hd / (H / G);
            double *S = (double *)malloc((size_t)per_state * sizeof(double));
            double *u = (double *)malloc((size_t)dv * sizeof(double));
            if (init && (has_init == NULL || has_init[s] != 0))
                memcpy(S, init + ((int64_t)s * H + hd) * per_state, (size_t)per_state * sizeof(double));
            else
                memset(S, 0, (size_t)per_state * sizeof(double));
            const int64_t t0 = cu_seqlens[s], t1 = cu_seqlens[s + 1];
            for (int64_t t = t0; t < t1; ++t) {
                const double a = exp(gate[t * H + hd]), b = beta[t * H + hd];
                const double *kt = k + (t * G + g) * dk, *qt = q + (t * G + g) * dk;
                const double *vt = v + (t * H + hd) * dv;
                for (int64_t i = 0; i < per_state; ++i)
                    S[i] *= a;
                for (int64_t c = 0; c < dv; ++c) {
                    double hk = 0.0;
                    for (int64_t r = 0; r < dk; ++r)
                        hk += S[c * dk + r] * kt[r];
                    u[c] = b * (vt[c] - hk);
                }
                for (int64_t c = 0; c < dv; ++c)
                    for (int64_t r = 0; r < dk; ++r)
                        S[c * dk + r] += u[c] * kt[r];
                double *ot = o + (t * H + hd) * dv;
                for (int64_t c = 0; c < dv; ++c) {
                    double acc = 0.0;
                    for (int64_t r = 0; r < dk; ++r)
                        acc += S[c * dk + r] * qt[r];
                    ot[c] = scale * acc;
                }
                const int64_t local = t - t0;
                if (chunk_states && chunk_size > 0 && ((local + 1) % chunk_size == 0 || t == t1 - 1)) {
                    const int64_t c = chunk_base[s] + local / chunk_size;
                    memcpy(chunk_states + (c * H + hd) * per_state, S, (size_t)per_state * sizeof(double));
                }
            }
            memcpy(final_states + ((int64_t)s * H + hd) * per_state, S, (size_t)per_state * sizeof(double));
            free(S);
            free(u);
        }
    }
    free(chunk_base);
    return 0;
}

/*
 * Prefill bites of the scheduler, one step (the prefix-caching page: the
 * scheduler diff fragment, which re-aligns a misaligned start at the next
 * boundary and otherwise clips the end down to a boundary, and the review
 * note under it, which re-aligns a misaligned start even on the final bite and
 * lets the final bite from an aligned start end anywhere).
 * Sequence s has prompt_len[s] tokens, num_computed_tokens[s] of them done,
 * and at most budget[s] tokens this step:
 *     last_aligned = floor(prompt_len / align) * align
 *     next         = (floor(start / align) + 1) * align     (start = num_computed_tokens)
 *     end          = min(start + budget, prompt_len)
 *     if start is not a multiple of align and next <= last_aligned:  end = min(end, next)
 *     else if end < last_aligned:                                    end = floor(end / align) * align
 *     num_scheduled[s] = end - start
 * So every bite ends on a multiple of align except the one that ends the
 * prompt, and only a misaligned starting position (state loaded from
 * elsewhere) can start a bite off the grid: it ends at the next boundary.
 * Returns 0, or -1 when align <= 0, a budget is below align, or a start lies
 * outside [0, prompt_len].
 */
int oracle_prefill_bites(int32_t nseqs, const int32_t *num_computed_tokens, const int32_t *prompt_len,
                         const int32_t *budget, int32_t align, int32_t *num_scheduled)
{
    if (align <= 0)
        return -1;
    for (int32_t s = 0; s < nseqs; ++s) {
        const int64_t start = num_computed_tokens[s], len = prompt_len[s];
        if (start < 0 || start > len || budget[s] < align)
            return -1;
        const int64_t last_aligned = len / align * align;
        const int64_t next = (start / align + 1) * align;
        int64_t end = start + budget[s] < len ? start + budget[s] : len;
        if (start % align != 0 && next <= last_aligned) {
            if (next < end)
                end = next;
        } else if (end < last_aligned) {
            end = end / align * align;
        }
        num_scheduled[s] = (int32_t)(end - start);
    }
    return 0;
}

/*
 * One decode step with dual state anchors. The prefix-caching page's decode
 * kernels read a request's running state from one cache slot (the previous
 * step's write anchor) and write the advanced state to another (the current
 * anchor), so that a cached checkpoint is never overwritten in place.
 * Here, for each sequence s (one new token each) and head h:
 *     S     = state_cache[read_slot[s], h]      (all zero when read_slot[s] < 0)
 *     delta = softplus(dt[s,h] + dt_bias[h])
 *     S'    = exp(A[h] * delta) * S + delta * x[s,h] (outer) B[s,g]
 *     y[s,h] = S' . C[s,g] + D[h] * x[s,h]
 *     state_cache[write_slot[s], h] = S'        (skipped when write_slot[s] < 0)
 * All slot reads happen before any slot write, so read_slot == write_slot is an
 * in-place update. Layouts: x, y (S,H,P); dt (S,H); B, C (S,G,N); cache
 * (num_slots,H,P,N). A sequence with a slot >= num_slots is skipped (y left
 * as is, nothing written) and the call returns -2; -1 on bad shapes.
 */
int oracle_ssd_decode(int32_t nseqs, int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                      const double *x, const double *dt, const double *dt_bias, const double *A,
                      const double *B, const double *C, const double *D, double *state_cache,
                      int32_t num_slots, const int32_t *read_slot, const int32_t *write_slot,
                      double *y)
{
    const int64_t H = nheads, P = headdim, N = dstate, G = ngroups;
    if (nseqs < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || num_slots < 0)
        return -1;
    const int64_t per_state = H * P * N;
    int bad = 0;
    /* gather every sequence's entering state first (reads before writes) */
    double *h_in = (double *)calloc((size_t)(nseqs > 0 ? nseqs : 1) * (size_t)per_state, sizeof(double));
    if (!h_in)
        return -1;
    for (int64_t s = 0; s < nseqs; ++s) {
        const int32_t r = read_slot ? read_slot[s] : -1;
        const int32_t w = write_slot ? write_slot[s] : -1;
        if (r >= num_slots || w >= num_slots) {
            bad = 1;
            continue;
        }
        if (r >= 0)
            memcpy(h_in + s * per_state, state_cache + (int64_t)r * per_state,
                   (size_t)per_state * sizeof(double));
    }
    for (int64_t s = 0; s < nseqs; ++s) {
        const int32_t r = read_slot ? read_slot[s] : -1;
        const int32_t w = write_slot ? write_slot[s] : -1;
        if (r >= num_slots || w >= num_slots)
            continue;
        for (int64_t hd = 0; hd < H; ++hd) {
            const int64_t g = hd / (H / G);
            const double delta = oracle_softplus(dt[s * H + hd] + (dt_bias ? dt_bias[hd] : 0.0));
            const double decay = exp(delta * A[hd]);
            const double *xs = x + (s * H + hd) * P;
            const double *Bs = B + (s * G + g) * N;
            const double *Cs = C + (s * G + g) * N;
            double *hs = h_in + s * per_state + hd * P * N;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    hs[p * N + n] = decay * hs[p * N + n] + delta * xs[p] * Bs[n];
                    acc += Cs[n] * hs[p * N + n];
                }
                y[(s * H + hd) * P + p] = acc + (D ? D[hd] : 0.0) * xs[p];
            }
        }
        if (w >= 0)
            memcpy(state_cache + (int64_t)w * per_state, h_in + s * per_state,
                   (size_t)per_state * sizeof(double));
    }
    free(h_in);
    return bad ? -2 : 0;
}

/*
 * Varlen causal conv1d (the causal_conv1d step that runs before the scan and
 * whose metadata the prefix-caching page builds together with the other batch
 * metadata). The pages name the kernel without giving its formula; this is the
 * standard depthwise causal convolution of the Mamba2 block, read plainly:
 * each channel c has its own `width` taps weight[c, 0..W-1] (tap W-1 on the
 * current token), the window never reaches across a sequence start, and the
 * W-1 inputs before a sequence's first token come from a conv-state cache slot
 * (dual anchors, as for the SSM state: read from read_slot[s], zero when < 0;
 * the sequence's last W-1 inputs are written to write_slot[s], skipped when < 0).
 * For sequence s with L tokens at rows cu[s] .. cu[s+1]-1 and j in [0, L):
 *     u_j      = x[cu[s] + j, c]                            (j >= 0)
 *     u_j      = conv_states[read_slot[s], W-1+j, c]        (-(W-1) <= j < 0)
 *     out[cu[s]+j, c] = act(bias[c] + sum_k weight[c,k] * u_{j-(W-1)+k})
 *     conv_states[write_slot[s], i, c] = u_{L-(W-1)+i}      (i = 0 .. W-2)
 * act = identity (silu = 0) or SiLU z / (1 + e^-z) (silu = 1). Layouts: x, out
 * (T, channels); weight (channels, W); bias (channels) or NULL; conv_states
 * (num_slots, W-1, channels). Every state read happens before any state write.
 * A sequence with a slot >= num_slots is skipped (its rows of out left as
 * they are, nothing written) and the call returns -2; -1 on bad shapes.
 */
int oracle_causal_conv1d(int32_t nseqs, const int32_t *cu_seqlens, int32_t channels, int32_t width,
                         const double *x, const double *weight, const double *bias, int32_t silu,
                         double *conv_states, int32_t num_slots, const int32_t *read_slot,
                         const int32_t *write_slot, double *out)
{
    const int64_t Cn = channels, W = width;
    if (nseqs < 0 || Cn <= 0 || W < 1 || num_slots < 0)
        return -1;
    for (int32_t s = 0; s < nseqs; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s])
            return -1;
    const int64_t per_slot = (W - 1) * Cn;
    int bad = 0;
    /* each sequence's W-1 leading inputs, gathered before any slot write */
    double *pre = (double *)calloc((size_t)(nseqs > 0 ? nseqs : 1) * (size_t)(per_slot > 0 ? per_slot : 1),
                                   sizeof(double));
    if (!pre)
        return -1;
    for (int32_t s = 0; s < nseqs; ++s) {
        const int32_t r = read_slot ? read_slot[s] : -1;
        const int32_t w = write_slot ? write_slot[s] : -1;
        if (r >= num_slots || w >= num_slots) {
            bad |= 1;
            continue;
        }
        if (r >= 0 && per_slot > 0)
            memcpy(pre + (int64_t)s * per_slot, conv_states + (int64_t)r * per_slot,
                   (size_t)per_slot * sizeof(double));
    }
    for (int32_t s = 0; s < nseqs; ++s) {
        const int32_t r = read_slot ? read_slot[s] : -1;
        const int32_t w = write_slot ? write_slot[s] : -1;
        if (r >= num_slots || w >= num_slots)
            continue;
        const int64_t t0 = cu_seqlens[s], L = cu_seqlens[s + 1] - cu_seqlens[s];
        const double *ps = pre + (int64_t)s * per_slot;
        for (int64_t j = 0; j < L; ++j) {   /* (rows outer: the memory order of x and out) */
            for (int64_t c = 0; c < Cn; ++c) {
                double z = bias ? bias[c] : 0.0;
                for (int64_t k = 0; k < W; ++k) {
                    const int64_t jj = j - (W - 1) + k;   /* input position of tap k */
                    const double u = jj >= 0 ? x[(t0 + jj) * Cn + c] : ps[(W - 1 + jj) * Cn + c];
                    z += weight[c * W + k] * u;
                }
                out[(t0 + j) * Cn + c] = silu ? z / (1.0 + exp(-z)) : z;
            }
        }
        for (int64_t c = 0; c < Cn; ++c) {
            if (w >= 0) {
                for (int64_t i = 0; i < W - 1; ++i) {
                    const int64_t jj = L - (W - 1) + i;
                    conv_states[(int64_t)w * per_slot + i * Cn + c] =
                        jj >= 0 ? x[(t0 + jj) * Cn + c] : ps[(W - 1 + jj) * Cn + c];
                }
            }
        }
    }
    free(pre);
    return bad ? -2 : 0;
}
