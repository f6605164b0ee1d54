// Varlen chunk metadata and block-checkpoint plan / scatter kernels.
//
// Metadata ("Mamba2 varlen and metadata refactor", Purpose): tokens of all
// requests are packed along one axis with cu_seqlens; the chunk grid restarts
// at every sequence start so that no chunk spans two sequences, and it is built
// once per batch on the device (no host synchronisation).
//
// Plan ("Automatic prefix caching for GDN hybrid models", block-checkpoint
// scatter fragment): the state at each cache-block end that falls inside the
// scheduled tokens goes to that block's slot, only when the computed prefix is
// chunk-aligned; the source chunk is kept inside the sequence's own chunks;
// the last touched block receives the final state. Here each chunk asks which
// block (if any) ends with it, which gives the slot its state is written to
// directly by the scan.
#include "ssd_internal.h"

namespace ssd {

namespace {

constexpr int kMetaThreads = 1024;

__device__ __forceinline__ int block_inclusive_scan(int v, int *warp_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    if (lane == 63) warp_tot[wave] = v;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += warp_tot[w];
    int total = 0;
    for (int w = 0; w < nwaves; ++w) total += warp_tot[w];
    __syncthreads();
    warp_tot[16] = total;   // read back by every thread before the next scan
    return v + before;
}

__global__ __launch_bounds__(kMetaThreads) void ssd_metadata_kernel(MetaArgs a) {
    __shared__ int warp_tot[17];
    __shared__ int bad;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int32_t *cu = a.cu_seqlens;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (int s = tid; s <= a.S; s += nt) {
        const int v = cu[s];
        const bool ok = (s == 0 ? v == 0 : true) && (s == a.S ? v == a.T : true) &&
                        (s < a.S ? cu[s + 1] >= v : true);
        if (!ok) bad = 1;
    }
    __syncthreads();
    if (bad) {
        if (tid == 0) atomicOr(a.error_flag, SSD_DATA_BAD_CU_SEQLENS);
        return;
    }
    // seq_chunk_start = exclusive prefix sum of ceil(len / cs)
    int carry = 0;
    for (int base = 0; base < a.S; base += nt) {
        const int s = base + tid;
        const int n = s < a.S ? (cu[s + 1] - cu[s] + a.cs - 1) / a.cs : 0;
        const int incl = block_inclusive_scan(n, warp_tot);
        if (s < a.S) a.seq_chunk_start[s] = carry + incl - n;
        __syncthreads();
        carry += warp_tot[16];
        __syncthreads();
    }
    const int nch = carry;
    if (tid == 0) {
        a.seq_chunk_start[a.S] = nch;
        *a.nchunks = nch;
        a.chunk_offsets[a.max_chunks] = a.T;
        if (nch > a.max_chunks) atomicOr(a.error_flag, SSD_DATA_TOO_MANY_CHUNKS);
    }
    __syncthreads();   // seq_chunk_start (global) visible to the whole workgroup
    for (int c = tid; c < a.max_chunks; c += nt) {
        int off = a.T, idx = -1;
        if (c < nch) {
            // last sequence whose first chunk is <= c (empty sequences own no chunk)
            int lo = 0, hi = a.S;   // invariant: start[lo] <= c < start[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (a.seq_chunk_start[mid] <= c) lo = mid; else hi = mid;
            }
            idx = lo;
            off = cu[lo] + (c - a.seq_chunk_start[lo]) * a.cs;
        }
        a.chunk_offsets[c] = off;
        a.chunk_seq_idx[c] = idx;
    }
    // work order: decreasing length, ties by index (rank by counting)
    for (int s = tid; s < a.S; s += nt) {
        const int Ls = cu[s + 1] - cu[s];
        int rank = 0;
        for (int u = 0; u < a.S; ++u) {
            const int Lu = cu[u + 1] - cu[u];
            rank += (Lu > Ls) || (Lu == Ls && u < s);
        }
        a.seq_order[rank] = s;
    }
}

__global__ void ssd_plan_kernel(PlanArgs a) {
    const int64_t nblk = (int64_t)a.S * a.max_blocks;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int32_t *cu = a.cu_seqlens, *start = a.seq_chunk_start;
    if (*a.error_flag & SSD_DATA_BAD_CU_SEQLENS) {   // metadata undefined: plan nothing
        if (i < nblk) a.ckpt_src[i] = -1;
        else if (i < nblk + a.max_chunks) a.chunk_state_dst[i - nblk] = -1;
        return;
    }
    if (i < nblk) {
        // source chunk of block k of sequence s
        const int s = (int)(i / a.max_blocks), k = (int)(i % a.max_blocks);
        const int64_t L = (int64_t)cu[s + 1] - cu[s];
        int src = -1;
        if (L > 0) {
            const int64_t nc = a.num_computed_tokens ? a.num_computed_tokens[s] : 0;
            const int64_t first = nc / a.block_size, last = (nc + L - 1) / a.block_size;
            const int lo = start[s], hi = start[s + 1] - 1;
            if (k == 0 && last >= a.max_blocks) atomicOr(a.error_flag, SSD_DATA_BAD_BLOCK);
            if (k == last) {
                src = hi;
            } else if (k >= first && k < last && nc % a.cs == 0) {
                int64_t c = lo + ((int64_t)(k + 1) * a.block_size - nc) / a.cs - 1;
                src = (int)(c < lo ? lo : (c > hi ? hi : c));
            }
        }
        a.ckpt_src[i] = src;
    } else if (i < nblk + a.max_chunks) {
        // destination slot of chunk c
        const int c = (int)(i - nblk);
        int dst = -1;
        const int s = c < *a.nchunks ? a.chunk_seq_idx[c] : -1;
        if (s >= 0 && s < a.S) {
            const int64_t L = (int64_t)cu[s + 1] - cu[s];
            const int64_t nc = a.num_computed_tokens ? a.num_computed_tokens[s] : 0;
            const int64_t lc = c - start[s];
            const int64_t end = nc + ((lc + 1) * a.cs < L ? (lc + 1) * a.cs : L);
            int64_t k = -1;
            if (c == start[s + 1] - 1) k = (nc + L - 1) / a.block_size;          // final state block
            else if (nc % a.cs == 0 && end % a.block_size == 0) k = end / a.block_size - 1;  // block end
            if (k >= a.max_blocks) {
                atomicOr(a.error_flag, SSD_DATA_BAD_BLOCK);
                k = -1;
            }
            if (k >= 0) {
                const int slot = a.block_table[(int64_t)s * a.max_blocks + k];
                if (slot >= a.num_slots) atomicOr(a.error_flag, SSD_DATA_BAD_SLOT);
                else if (slot >= 0) dst = slot;
            }
        }
        a.chunk_state_dst[c] = dst;
    }
}

// state_cache[block_table[s][k]] = chunk_states[ckpt_src[s][k]] (one block row of
// the grid per (s, k), float4 copies along the state)
__global__ void ssd_scatter_kernel(PlanArgs a) {
    const int64_t i = blockIdx.x;   // (s, k)
    const int src = a.ckpt_src[i];
    const int slot = a.block_table[i];
    if (src < 0 || slot < 0 || slot >= a.num_slots || src >= a.max_chunks) return;
    const int64_t n4 = a.state_elems / 4;
    const float4 *from = reinterpret_cast<const float4 *>(a.chunk_states + (int64_t)src * a.state_elems);
    float4 *to = reinterpret_cast<float4 *>(a.state_cache + (int64_t)slot * a.state_elems);
    for (int64_t e = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; e < n4; e += (int64_t)gridDim.y * blockDim.x)
        to[e] = from[e];
}

}  // namespace

hipError_t launch_metadata(const MetaArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(ssd_metadata_kernel, dim3(1), dim3(kMetaThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs &a, hipStream_t stream) {
    const int64_t items = (int64_t)a.S * a.max_blocks + a.max_chunks;
    if (items > 0) {
        hipLaunchKernelGGL(ssd_plan_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.chunk_states != nullptr && (int64_t)a.S * a.max_blocks > 0) {
        const int64_t n4 = a.state_elems / 4;
        const unsigned gy = (unsigned)((n4 + 255) / 256 < 64 ? (n4 + 255) / 256 : 64);
        hipLaunchKernelGGL(ssd_scatter_kernel, dim3((unsigned)((int64_t)a.S * a.max_blocks), gy > 0 ? gy : 1),
                           dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace ssd
