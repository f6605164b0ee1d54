// C ABI of libssd.so: argument validation and launches (declarations and
// contracts in include/ssd.h). Every argument error is reported before
// anything is enqueued; the library never synchronises the host.
#include <stdint.h>

#include "ssd_internal.h"

namespace {

bool pow2_chunk(int32_t cs) { return cs >= 16 && cs <= 256 && (cs & (cs - 1)) == 0; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ssd_status check_meta(const ssd_varlen_meta *m) {
    if (m == nullptr || m->cu_seqlens == nullptr || m->chunk_offsets == nullptr ||
        m->chunk_seq_idx == nullptr || m->seq_chunk_start == nullptr || m->nchunks == nullptr ||
        m->seq_order == nullptr || m->error_flag == nullptr)
        return SSD_ERR_NULL_ARG;
    if (m->nseqs < 0 || m->total_tokens < 0 || m->max_chunks < 0) return SSD_ERR_SHAPE;
    if (!pow2_chunk(m->chunk_size)) return SSD_ERR_CHUNK_SIZE;
    // every sequence adds at most one partial chunk to T / chunk_size full ones
    if ((int64_t)m->max_chunks < (int64_t)m->total_tokens / m->chunk_size + m->nseqs) return SSD_ERR_CAPACITY;
    return SSD_OK;
}

}  // namespace

extern "C" {

const char *ssd_status_string(ssd_status status) {
    switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL_ARG: return "a required pointer is NULL";
    case SSD_ERR_CHUNK_SIZE: return "chunk_size must be a power of two in [16, 256]";
    case SSD_ERR_SHAPE: return "invalid sizes, nheads % ngroups != 0, or a pointer not 16-byte aligned";
    case SSD_ERR_BLOCK_SIZE: return "block_size must be a positive multiple of chunk_size";
    case SSD_ERR_CAPACITY: return "capacity below the required bound (max_chunks or chunk_states)";
    case SSD_ERR_DTYPE: return "unknown dtype";
    case SSD_ERR_HIP: return "a HIP call failed";
    case SSD_ERR_UNSUPPORTED: return "unsupported dtype/shape combination (headdim, dstate, dk, dv or chunk size)";
    }
    return "unknown status";
}

ssd_status ssd_varlen_metadata(const ssd_varlen_meta *meta, void *stream) {
    const ssd_status st = check_meta(meta);
    if (st != SSD_OK) return st;
    ssd::MetaArgs a{meta->cu_seqlens, meta->chunk_offsets, meta->chunk_seq_idx, meta->seq_chunk_start,
                    meta->nchunks, meta->seq_order, meta->error_flag, meta->nseqs, meta->total_tokens,
                    meta->chunk_size, meta->max_chunks};
    return ssd::launch_metadata(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_chunk_scan_varlen(const void *x, const float *dt, const float *dt_bias, const float *A,
                                 const void *B, const void *C, const float *D, ssd_dtype in_dtype,
                                 const ssd_varlen_meta *meta, int32_t nheads, int32_t headdim,
                                 int32_t dstate, int32_t ngroups, const float *initial_states,
                                 const int32_t *has_initial_state, void *y, float *final_states,
                                 float *chunk_states, const int32_t *chunk_state_dst,
                                 int32_t chunk_states_capacity, void *stream) {
    ssd_status st = check_meta(meta);
    if (st != SSD_OK) return st;
    if (in_dtype != SSD_F32 && in_dtype != SSD_BF16) return SSD_ERR_DTYPE;
    const bool empty = meta->total_tokens == 0;
    if ((!empty && (x == nullptr || dt == nullptr || B == nullptr || C == nullptr || y == nullptr)) ||
        A == nullptr || (meta->nseqs > 0 && final_states == nullptr))
        return SSD_ERR_NULL_ARG;
    if (nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 || nheads % ngroups != 0)
        return SSD_ERR_SHAPE;
    if (headdim % 16 != 0) return SSD_ERR_UNSUPPORTED;
    const bool n_ok = dstate == 16 || dstate == 32 || dstate == 64 || dstate == 128 ||
                      (dstate == 256 && in_dtype == SSD_BF16);
    if (!n_ok) return SSD_ERR_UNSUPPORTED;
    if (chunk_states != nullptr) {
        if (chunk_states_capacity <= 0) return SSD_ERR_CAPACITY;
        if (chunk_state_dst == nullptr && chunk_states_capacity < meta->max_chunks) return SSD_ERR_CAPACITY;
    }
    for (const void *p : {x, B, C, (const void *)y, (const void *)final_states, (const void *)initial_states,
                          (const void *)chunk_states})
        if (p != nullptr && !aligned16(p)) return SSD_ERR_SHAPE;

    ssd::ScanArgs a{};
    a.x = x; a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.B = B; a.C = C; a.D = D;
    a.init = initial_states; a.has_init = has_initial_state;
    a.y = y; a.final_states = final_states; a.chunk_states = chunk_states;
    a.chunk_state_dst = chunk_state_dst;
    a.cu_seqlens = meta->cu_seqlens; a.seq_chunk_start = meta->seq_chunk_start;
    a.seq_order = meta->seq_order; a.error_flag = meta->error_flag;
    a.T = meta->total_tokens; a.S = meta->nseqs; a.H = nheads; a.P = headdim; a.G = ngroups;
    a.cs = meta->chunk_size; a.max_chunks = meta->max_chunks;
    a.capacity = chunk_states ? chunk_states_capacity : 0;
    // headdim tile per workgroup: 64 columns when it divides headdim (4 waves,
    // or 8 with the state split between wave pairs for bf16 with dstate 128),
    // else 32 (2 waves) or 16 (1 wave)
    const int waves = headdim % 64 == 0 ? 4 : (headdim % 32 == 0 ? 2 : 1);
    const bool split = in_dtype == SSD_BF16 && dstate == 128 && headdim % 64 == 0;
    a.nptiles = headdim / (16 * waves);
    a.xcd_mode = ssd::xcd_mode_for(meta->nseqs, nheads, ngroups, a.nptiles);
    // the warp-specialised kernel walks 64-token tiles (chunk_size >= 64), of
    // one head or of a.items heads per workgroup
    const bool ws = split && meta->chunk_size >= 64;
    const int64_t wgs = (int64_t)meta->nseqs * nheads * a.nptiles;
    a.items = ws ? ssd::ws_items_for(a.xcd_mode, wgs, nheads / ngroups)
                 : split ? ssd::split_items_for(a.xcd_mode, wgs, nheads / ngroups) : 1;
    if (meta->nseqs == 0) return SSD_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = ws ? ssd::launch_scan_ws_bf16(a, dstate, s)
                         : split ? ssd::launch_scan_split_bf16(a, dstate, s)
                         : in_dtype == SSD_BF16 ? ssd::launch_scan_bf16(a, waves, dstate, s)
                                                : ssd::launch_scan_f32(a, waves, dstate, s);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_export_chunk_states(const ssd_varlen_meta *meta, const int32_t *num_computed_tokens,
                                   const int32_t *block_table, int32_t max_blocks_per_seq,
                                   int32_t block_size, int32_t *ckpt_src, int32_t *chunk_state_dst,
                                   const float *chunk_states, int32_t state_elems, float *state_cache,
                                   int32_t num_slots, void *stream) {
    ssd_status st = check_meta(meta);
    if (st != SSD_OK) return st;
    if (max_blocks_per_seq < 0 || num_slots < 0) return SSD_ERR_SHAPE;
    if ((meta->nseqs > 0 && max_blocks_per_seq > 0 && (block_table == nullptr || ckpt_src == nullptr)) ||
        (meta->max_chunks > 0 && chunk_state_dst == nullptr))
        return SSD_ERR_NULL_ARG;
    if (block_size <= 0 || block_size % meta->chunk_size != 0) return SSD_ERR_BLOCK_SIZE;
    if (chunk_states != nullptr) {
        if (state_cache == nullptr) return SSD_ERR_NULL_ARG;
        if (state_elems <= 0 || state_elems % 4 != 0) return SSD_ERR_SHAPE;
        if (!aligned16(chunk_states) || !aligned16(state_cache)) return SSD_ERR_SHAPE;
    }
    ssd::PlanArgs a{};
    a.cu_seqlens = meta->cu_seqlens; a.seq_chunk_start = meta->seq_chunk_start;
    a.chunk_seq_idx = meta->chunk_seq_idx; a.nchunks = meta->nchunks;
    a.num_computed_tokens = num_computed_tokens; a.block_table = block_table;
    a.ckpt_src = ckpt_src; a.chunk_state_dst = chunk_state_dst; a.error_flag = meta->error_flag;
    a.chunk_states = chunk_states; a.state_cache = state_cache;
    a.S = meta->nseqs; a.cs = meta->chunk_size; a.max_chunks = meta->max_chunks;
    a.max_blocks = max_blocks_per_seq; a.block_size = block_size; a.state_elems = state_elems;
    a.num_slots = num_slots;
    return ssd::launch_plan(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_decode_step(const void *x, const float *dt, const float *dt_bias, const float *A,
                           const void *B, const void *C, const float *D, ssd_dtype in_dtype,
                           int32_t nseqs, int32_t nheads, int32_t headdim, int32_t dstate,
                           int32_t ngroups, float *state_cache, int32_t num_slots,
                           const int32_t *read_slot, const int32_t *write_slot, void *y,
                           int32_t *error_flag, void *stream) {
    if (in_dtype != SSD_F32 && in_dtype != SSD_BF16) return SSD_ERR_DTYPE;
    if (nseqs < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
        nheads % ngroups != 0 || num_slots < 0)
        return SSD_ERR_SHAPE;
    if (!(dstate == 16 || dstate == 32 || dstate == 64 || dstate == 128 || dstate == 256))
        return SSD_ERR_UNSUPPORTED;
    if (A == nullptr) return SSD_ERR_NULL_ARG;
    if (nseqs > 0 && (x == nullptr || dt == nullptr || B == nullptr || C == nullptr || y == nullptr ||
                      state_cache == nullptr || read_slot == nullptr || write_slot == nullptr))
        return SSD_ERR_NULL_ARG;
    if (state_cache != nullptr && !aligned16(state_cache)) return SSD_ERR_SHAPE;
    ssd::DecodeArgs a{};
    a.x = x; a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.B = B; a.C = C; a.D = D;
    a.cache = state_cache; a.read_slot = read_slot; a.write_slot = write_slot; a.y = y;
    a.error_flag = error_flag;
    a.S = nseqs; a.H = nheads; a.P = headdim; a.G = ngroups; a.num_slots = num_slots;
    a.pchunks = ssd::decode_pchunks(headdim, dstate);
    return ssd::launch_decode(a, in_dtype == SSD_BF16, dstate, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_causal_conv1d_varlen(const void *x, const float *weight, const float *bias,
                                    ssd_dtype in_dtype, const ssd_varlen_meta *meta, int32_t channels,
                                    int32_t width, int32_t activation, void *conv_states,
                                    int32_t num_slots, const int32_t *read_slot,
                                    const int32_t *write_slot, void *out, void *stream) {
    ssd_status st = check_meta(meta);
    if (st != SSD_OK) return st;
    if (in_dtype != SSD_F32 && in_dtype != SSD_BF16) return SSD_ERR_DTYPE;
    if (channels <= 0 || num_slots < 0) return SSD_ERR_SHAPE;
    if (channels % 8 != 0 || width < 1 || width > 4 || (activation != 0 && activation != 1))
        return SSD_ERR_UNSUPPORTED;
    if (weight == nullptr || (meta->total_tokens > 0 && (x == nullptr || out == nullptr)))
        return SSD_ERR_NULL_ARG;
    if (width > 1 && num_slots > 0 && (read_slot != nullptr || write_slot != nullptr) && conv_states == nullptr)
        return SSD_ERR_NULL_ARG;
    for (const void *p : {x, (const void *)out, (const void *)conv_states})
        if (p != nullptr && !aligned16(p)) return SSD_ERR_SHAPE;
    ssd::Conv1dArgs a{};
    a.x = x; a.weight = weight; a.bias = bias; a.out = out; a.states = conv_states;
    a.read_slot = read_slot; a.write_slot = write_slot;
    a.chunk_offsets = meta->chunk_offsets; a.chunk_seq_idx = meta->chunk_seq_idx;
    a.seq_chunk_start = meta->seq_chunk_start; a.error_flag = meta->error_flag;
    a.S = meta->nseqs; a.C = channels; a.W = width; a.num_slots = (conv_states != nullptr || width == 1) ? num_slots : 0;   // (width 1 keeps no rows)
    a.max_chunks = meta->max_chunks; a.channel_blocks = ssd::conv1d_channel_blocks(channels);
    a.silu = activation;
    return ssd::launch_conv1d(a, in_dtype == SSD_BF16, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SSD_OK : SSD_ERR_HIP;
}

size_t ssd_gated_delta_workspace_size(int32_t max_chunks, int32_t nheads) {
    if (max_chunks <= 0 || nheads <= 0) return 0;
    return (size_t)max_chunks * (size_t)nheads * ssd::kGdnWsBytes;
}

ssd_status ssd_gated_delta_chunk_varlen(const void *q, const void *k, const void *v, const float *gate,
                                        const float *beta, float scale, ssd_dtype in_dtype,
                                        const ssd_varlen_meta *meta, int32_t nheads, int32_t nkheads, int32_t dk,
                                        int32_t dv, const float *initial_states, const int32_t *has_initial_state,
                                        void *o, float *final_states, float *chunk_states,
                                        const int32_t *chunk_state_dst, int32_t chunk_states_capacity,
                                        void *workspace, size_t workspace_bytes, void *stream) {
    ssd_status st = check_meta(meta);
    if (st != SSD_OK) return st;
    if (in_dtype != SSD_F32 && in_dtype != SSD_BF16) return SSD_ERR_DTYPE;
    const bool empty = meta->total_tokens == 0;
    if ((!empty && (q == nullptr || k == nullptr || v == nullptr || gate == nullptr || beta == nullptr ||
                    o == nullptr)) ||
        (meta->nseqs > 0 && final_states == nullptr))
        return SSD_ERR_NULL_ARG;
    if (nheads <= 0 || nkheads <= 0 || dk <= 0 || dv <= 0 || nheads % nkheads != 0) return SSD_ERR_SHAPE;
    if (in_dtype != SSD_BF16 || dk != 128 || dv % 64 != 0 || meta->chunk_size != 64) return SSD_ERR_UNSUPPORTED;
    if (chunk_states != nullptr) {
        if (chunk_states_capacity <= 0) return SSD_ERR_CAPACITY;
        if (chunk_state_dst == nullptr && chunk_states_capacity < meta->max_chunks) return SSD_ERR_CAPACITY;
    }
    if (!empty && (workspace == nullptr || workspace_bytes < ssd_gated_delta_workspace_size(meta->max_chunks, nheads)))
        return SSD_ERR_CAPACITY;
    for (const void *p : {q, k, v, (const void *)o, (const void *)final_states, (const void *)initial_states,
                          (const void *)chunk_states, (const void *)workspace})
        if (p != nullptr && !aligned16(p)) return SSD_ERR_SHAPE;
    ssd::GdnArgs a{};
    a.q = static_cast<const uint16_t *>(q); a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v); a.gate = gate; a.beta = beta;
    a.init = initial_states; a.has_init = has_initial_state;
    a.o = static_cast<uint16_t *>(o); a.final_states = final_states;
    a.chunk_states = chunk_states; a.chunk_state_dst = chunk_state_dst;
    a.workspace = static_cast<uint16_t *>(workspace);
    a.cu_seqlens = meta->cu_seqlens; a.seq_chunk_start = meta->seq_chunk_start; a.seq_order = meta->seq_order;
    a.chunk_offsets = meta->chunk_offsets; a.chunk_seq_idx = meta->chunk_seq_idx;
    a.error_flag = meta->error_flag; a.scale = scale;
    a.T = meta->total_tokens; a.S = meta->nseqs; a.H = nheads; a.G = nkheads; a.dv = dv;
    a.max_chunks = meta->max_chunks; a.capacity = chunk_states ? chunk_states_capacity : 0;
    a.nptiles = dv / 64;
    if (meta->nseqs == 0) return SSD_OK;
    return ssd::launch_gdn(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_gated_delta_chunk_varlen_noalloc(const void *q, const void *k, const void *v, const float *gate,
                                                const float *beta, float scale, ssd_dtype in_dtype,
                                                const ssd_varlen_meta *meta, int32_t nheads, int32_t nkheads,
                                                int32_t dk, int32_t dv, const float *initial_states,
                                                const int32_t *has_initial_state, void *o, float *final_states,
                                                float *chunk_states, const int32_t *chunk_state_dst,
                                                int32_t chunk_states_capacity, void *stream) {
    const ssd_status st = check_meta(meta);
    if (st != SSD_OK) return st;
    const size_t need = meta->total_tokens > 0 ? ssd_gated_delta_workspace_size(meta->max_chunks, nheads) : 0;
    if (need > ssd::kGdnScratchBytes) return SSD_ERR_CAPACITY;
    void *ws = nullptr;
    if (need > 0 && ssd::gdn_scratch(&ws) != hipSuccess) return SSD_ERR_HIP;
    return ssd_gated_delta_chunk_varlen(q, k, v, gate, beta, scale, in_dtype, meta, nheads, nkheads, dk, dv,
                                        initial_states, has_initial_state, o, final_states, chunk_states,
                                        chunk_state_dst, chunk_states_capacity, ws, ws ? ssd::kGdnScratchBytes : 0,
                                        stream);
}

ssd_status ssd_prefill_bites(int32_t nseqs, const int32_t *num_computed_tokens, const int32_t *prompt_len,
                             const int32_t *budget, int32_t align, int32_t *num_scheduled) {
    if (nseqs < 0 || align <= 0) return SSD_ERR_SHAPE;
    if (nseqs > 0 && (num_computed_tokens == nullptr || prompt_len == nullptr || budget == nullptr ||
                      num_scheduled == nullptr))
        return SSD_ERR_NULL_ARG;
    for (int32_t s = 0; s < nseqs; ++s)
        if (num_computed_tokens[s] < 0 || num_computed_tokens[s] > prompt_len[s] || budget[s] < align)
            return SSD_ERR_SHAPE;
    for (int32_t s = 0; s < nseqs; ++s) {
        const int64_t pos = num_computed_tokens[s], total = prompt_len[s];
        const int64_t grid_end = total - total % align;            // last block boundary of the prompt
        const int64_t boundary = pos - pos % align + align;        // first boundary after pos
        const int64_t want = pos + budget[s];
        int64_t stop = want < total ? want : total;
        if (pos % align != 0) {
            if (boundary <= grid_end && boundary < stop) stop = boundary;   // back onto the grid
        } else if (stop < grid_end) {
            stop -= stop % align;                                           // end on the grid
        }
        num_scheduled[s] = (int32_t)(stop - pos);
    }
    return SSD_OK;
}

}  // extern "C"
