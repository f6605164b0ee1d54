// Internal interface between the C-ABI host code (ssd_api.hip) and the kernel
// translation units of libssd.so. Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssd.h"

namespace ssd {

// Arguments of the fused chunk-walk scan kernel (one workgroup per
// (sequence, head, headdim tile), walking the sequence's chunks in order).
struct ScanArgs {
    const void *x;
    const float *dt;
    const float *dt_bias;   // nullable
    const float *A;
    const void *B;
    const void *C;
    const float *D;         // nullable
    const float *init;      // nullable
    const int32_t *has_init;  // nullable
    void *y;
    float *final_states;
    float *chunk_states;      // nullable
    const int32_t *chunk_state_dst;  // nullable
    const int32_t *cu_seqlens;
    const int32_t *seq_chunk_start;
    const int32_t *seq_order;
    int32_t *error_flag;
    int32_t T, S, H, P, G, cs, max_chunks, capacity, nptiles;
    // workgroup -> XCD mapping (see decode_block): one of the kXcd* values
    int32_t xcd_mode;
    // consecutive heads walked by one workgroup (split-state kernel; 1 = one head)
    int32_t items;
};

enum : int32_t { kXcdNone = 0, kXcdPairs = 1, kXcdSplit = 2, kXcdPairsIfEqual = 3, kXcdPairsIfEqualElseNone = 4 };

// Mapping for a launch: pairs when that balances the XCDs whatever the lengths
// (G a multiple of 8); else pairs only where the lengths turn out equal
// (checked on the device), and otherwise an even split of every sequence
// across the XCDs, or block order where the split does not divide.
inline int32_t xcd_mode_for(int32_t nseqs, int32_t nheads, int32_t ngroups, int32_t nptiles) {
    const bool pairs = (int64_t)nseqs * ngroups % 8 == 0;
    const bool split = (int64_t)nheads * nptiles % 8 == 0;
    if (pairs && ngroups % 8 == 0) return kXcdPairs;
    if (pairs) return split ? kXcdPairsIfEqual : kXcdPairsIfEqualElseNone;
    return split ? kXcdSplit : kXcdNone;
}

// Heads walked by one workgroup of the split-state kernel: with the pair
// mapping and at least 16 workgroups per CU (256 CUs) to begin with, merge
// heads of one (sequence, group) pair so that each workgroup walks 2 or 4 of
// them as one tile stream, keeping at least 8 workgroups per CU.
inline int32_t split_items_for(int32_t xcd_mode, int64_t blocks, int32_t heads_per_group) {
    if (xcd_mode != kXcdPairs) return 1;
    for (int32_t k : {4, 2})
        if (heads_per_group % k == 0 && blocks / k >= 2048) return k;
    return 1;
}

// The same for the warp-specialised kernel, whose pipeline runs on from one
// head into the next: up to 8 heads per workgroup, keeping at least 4
// workgroups per CU (on the 64-sequence batch 8 heads timed 2 % faster than
// 4, 16 heads 1 % slower).
inline int32_t ws_items_for(int32_t xcd_mode, int64_t blocks, int32_t heads_per_group) {
    if (xcd_mode != kXcdPairs) return 1;
    for (int32_t k : {8, 4, 2})
        if (heads_per_group % k == 0 && blocks / k >= 1024) return k;
    return 1;
}

// Launches the scan for one (dtype, waves-per-workgroup, dstate) instance.
hipError_t launch_scan_bf16(const ScanArgs &a, int waves, int dstate, hipStream_t stream);
hipError_t launch_scan_f32(const ScanArgs &a, int waves, int dstate, hipStream_t stream);
// Split-state bf16 scan (eight waves per 64 headdim columns; dstate 128).
hipError_t launch_scan_split_bf16(const ScanArgs &a, int dstate, hipStream_t stream);
// Warp-specialised bf16 scan (four chain and four helper waves per 64 headdim
// columns; dstate 128, chunk_size >= 64, one head per workgroup).
hipError_t launch_scan_ws_bf16(const ScanArgs &a, int dstate, hipStream_t stream);

// Decode step with dual state anchors (one token per sequence).
struct DecodeArgs {
    const void *x;            // (S, H, P) bf16 or f32
    const float *dt;          // (S, H)
    const float *dt_bias;     // nullable
    const float *A;
    const void *B, *C;        // (S, G, N)
    const float *D;           // nullable
    float *cache;             // (num_slots, H, P, N)
    const int32_t *read_slot, *write_slot;   // (S)
    void *y;                  // (S, H, P)
    int32_t *error_flag;      // nullable
    int32_t S, H, P, G, num_slots, pchunks;
};
int32_t decode_pchunks(int32_t headdim, int32_t dstate);   // workgroups per (sequence, head)

// Varlen causal conv1d over the scan's chunk grid (see ssd_conv1d.hip).
struct Conv1dArgs {
    const void *x;            // (T, C) bf16 or f32
    const float *weight;      // (C, W)
    const float *bias;        // (C) or null
    void *out;                // (T, C), element type of x
    void *states;             // (num_slots, W-1, C), element type of x
    const int32_t *read_slot, *write_slot;   // (S) or null (= all -1)
    const int32_t *chunk_offsets, *chunk_seq_idx, *seq_chunk_start;   // the batch's chunk grid
    int32_t *error_flag;
    int32_t S, C, W, num_slots, max_chunks, channel_blocks, silu;
};
int32_t conv1d_channel_blocks(int32_t channels);   // workgroups per chunk
hipError_t launch_conv1d(const Conv1dArgs &a, bool bf16, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, bool bf16, int dstate, hipStream_t stream);

// Chunked gated delta rule (see ssd_gdn.hip).
constexpr int kGdnWsBytes = 64 * 64 * 2;   // workspace per (chunk, value head): T (64 x 64 bf16)
struct GdnArgs {
    const uint16_t *q, *k, *v;          // (T,G,dk), (T,G,dk), (T,H,dv) bf16
    const float *gate, *beta;           // (T,H)
    const float *init;                  // (S,H,dv,dk) or null
    const int32_t *has_init;            // (S) or null
    uint16_t *o;                        // (T,H,dv) bf16
    float *final_states;                // (S,H,dv,dk)
    float *chunk_states;                // checkpoint cache or null
    const int32_t *chunk_state_dst;     // slot per chunk or null (-> chunk index)
    uint16_t *workspace;                // (max_chunks, H, 64, 64) bf16
    const int32_t *cu_seqlens, *seq_chunk_start, *seq_order, *chunk_offsets, *chunk_seq_idx;
    int32_t *error_flag;
    float scale;
    int32_t T, S, H, G, dv, max_chunks, capacity, nptiles;
};
hipError_t launch_gdn(const GdnArgs &a, hipStream_t stream);
// The allocation-free variant's static workspace (per device) and its size.
constexpr size_t kGdnScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
hipError_t gdn_scratch(void **ptr);

struct MetaArgs {
    const int32_t *cu_seqlens;
    int32_t *chunk_offsets, *chunk_seq_idx, *seq_chunk_start, *nchunks, *seq_order, *error_flag;
    int32_t S, T, cs, max_chunks;
};
hipError_t launch_metadata(const MetaArgs &a, hipStream_t stream);

struct PlanArgs {
    const int32_t *cu_seqlens, *seq_chunk_start, *chunk_seq_idx, *nchunks;
    const int32_t *num_computed_tokens;  // nullable
    const int32_t *block_table;
    int32_t *ckpt_src, *chunk_state_dst, *error_flag;
    const float *chunk_states;  // nullable: scatter now
    float *state_cache;
    int32_t S, cs, max_chunks, max_blocks, block_size, state_elems, num_slots;
};
hipError_t launch_plan(const PlanArgs &a, hipStream_t stream);

}  // namespace ssd
