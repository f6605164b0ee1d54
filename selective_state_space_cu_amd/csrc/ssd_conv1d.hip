// Varlen causal conv1d with a conv-state cache: the depthwise causal
// convolution that runs before the scan (the causal_conv1d kernel of the
// prefix-caching page, whose metadata is built with the rest of the batch
// metadata; here it walks the scan's own chunk grid). For sequence s, token j
// of its L tokens and channel c:
//   u_j  = x[cu[s]+j, c]                          (j >= 0)
//   u_j  = states[read_slot[s], W-1+j, c]         (-(W-1) <= j < 0; zero if read_slot[s] < 0)
//   out[cu[s]+j, c] = act(bias[c] + sum_k w[c,k] u_{j-(W-1)+k})     (act: identity or SiLU)
//   states[write_slot[s], i, c] = u_{L-(W-1)+i}   (i < W-1; skipped if write_slot[s] < 0)
//
// Memory-bound: every input row is read once and every output row written once
// (plus W-1 halo rows per chunk). One workgroup per (chunk, 1024-channel block):
// each lane owns 8 consecutive channels (16-byte bf16 vectors, so a wave reads
// and writes whole 1 KB row segments), walks the chunk's tokens in order and
// keeps the last W-1 inputs in registers. Row loads run one group of
// 16 (bf16) or 8 (fp32) tokens ahead of the arithmetic (double-buffered, still packed).
// The chunk that starts a sequence seeds its window from the read slot; the
// chunk that ends it writes the window to the write slot. Empty
// sequences own no chunk: extra workgroups after the chunk grid copy their
// state (or zeros) from the read slot to the write slot.
#include "ssd_scan.hpp"

namespace ssd {

constexpr int kConvThreads = 128;   // 1024 channels per workgroup
constexpr int kConvVec = 8;         // channels per lane
// token rows per group (a group in flight while the previous one is computed):
// 16 packed bf16 rows (4 VGPRs each) timed 2-3 % faster than 8; fp32 rows take
// 8 VGPRs each and keep 8
template <typename T> constexpr int kConvUnrollOf = sizeof(T) == 2 ? 16 : 8;

template <typename T> struct ConvIO;

template <> struct ConvIO<__bf16> {
    using Raw = u32x4;   // 8 packed bf16
    __device__ static Raw raw(const void *__restrict__ base, int64_t elem) {
        return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(base) + elem);
    }
    __device__ static void unpack(const Raw &w, float (&v)[kConvVec]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    }
    __device__ static void load(const void *base, int64_t elem, float (&v)[kConvVec]) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(base) + elem);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    }
    __device__ static void store(void *base, int64_t elem, const float (&v)[kConvVec], bool nt) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16(v[2 * i], v[2 * i + 1]);
        u32x4 *p = reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(base) + elem);
        if (nt) __builtin_nontemporal_store(w, p);
        else *p = w;
    }
};

template <> struct ConvIO<float> {
    struct Raw { f32x4 a, b; };
    __device__ static Raw raw(const void *__restrict__ base, int64_t elem) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(base) + elem);
        return Raw{p[0], p[1]};
    }
    __device__ static void unpack(const Raw &w, float (&v)[kConvVec]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = w.a[i];
            v[4 + i] = w.b[i];
        }
    }
    __device__ static void load(const void *base, int64_t elem, float (&v)[kConvVec]) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(base) + elem);
        const f32x4 a = p[0], b = p[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = a[i];
            v[4 + i] = b[i];
        }
    }
    __device__ static void store(void *base, int64_t elem, const float (&v)[kConvVec], bool nt) {
        f32x4 *p = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(base) + elem);
        const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        if (nt) {
            __builtin_nontemporal_store(a, p);
            __builtin_nontemporal_store(b, p + 1);
        } else {
            p[0] = a;
            p[1] = b;
        }
    }
};

// SiLU z / (1 + e^-z) with the hardware exp2 and reciprocal (about 1 ulp each;
// for large |z| the error stays below 2^-23 |z|, under the bias + taps magnitude)
__device__ __forceinline__ float silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

template <typename T, int W>
__global__ __launch_bounds__(kConvThreads) void ssd_conv1d_kernel(Conv1dArgs a) {
    constexpr int WR = W > 1 ? W - 1 : 1;   // window rows (at least one, unused when W = 1)
    using IO = ConvIO<T>;
    const int nxb = a.channel_blocks;
    const int cb = blockIdx.x % nxb, row = blockIdx.x / nxb;
    const int ch = (cb * kConvThreads + threadIdx.x) * kConvVec;
    if (ch >= a.C) return;
    if (__builtin_nontemporal_load(a.error_flag) & SSD_DATA_BAD_CU_SEQLENS) return;

    // which sequence, and (for a chunk) which tokens
    int s, t0 = 0, t1 = 0;
    bool first = true, last = true;
    if (row < a.max_chunks) {
        const int c = row;
        s = a.chunk_seq_idx[c];
        if (s < 0) return;   // past the last chunk
        t0 = a.chunk_offsets[c];
        t1 = a.chunk_offsets[c + 1];
        first = c == a.seq_chunk_start[s];
        last = c == a.seq_chunk_start[s + 1] - 1;
    } else {
        s = row - a.max_chunks;   // empty-sequence row
        if (a.seq_chunk_start[s + 1] != a.seq_chunk_start[s]) return;
    }
    const int rs = a.read_slot != nullptr ? a.read_slot[s] : -1;
    const int ws = a.write_slot != nullptr ? a.write_slot[s] : -1;
    // refused (nothing of the sequence read or written): a slot past the cache, or
    // one slot read and written by a sequence of several chunks, whose last
    // chunk could overwrite it before the first chunk has read it
    const bool in_place_multi = rs >= 0 && rs == ws && a.seq_chunk_start[s + 1] - a.seq_chunk_start[s] > 1;
    if (rs >= a.num_slots || ws >= a.num_slots || in_place_multi) {
        if (ch == 0 && first) atomicOr(a.error_flag, SSD_DATA_BAD_SLOT);
        return;
    }
    const int64_t C = a.C;
    const int64_t slot_elems = (int64_t)(W - 1) * C;

    // the W-1 inputs before the chunk's first token
    float win[WR][kConvVec];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
        if (!first) IO::load(a.x, (int64_t)(t0 - (W - 1) + i) * C + ch, win[i]);
        else if (rs >= 0) IO::load(a.states, rs * slot_elems + i * C + ch, win[i]);
        else {
#pragma unroll
            for (int v = 0; v < kConvVec; ++v) win[i][v] = 0.0f;
        }
    }

    if (t1 > t0) {
        float w[W][kConvVec], bias[kConvVec];
#pragma unroll
        for (int v = 0; v < kConvVec; ++v) {
#pragma unroll
            for (int k = 0; k < W; ++k) w[k][v] = a.weight[(int64_t)(ch + v) * W + k];
            bias[v] = a.bias != nullptr ? a.bias[ch + v] : 0.0f;
        }
        // rows in groups of kConvUnroll, the next group's loads issued before
        // the current group's arithmetic and stores (packed until used)
        const void *__restrict__ xs = a.x;
        void *__restrict__ os = a.out;
        constexpr int kConvUnroll = kConvUnrollOf<T>;
        typename IO::Raw cur[kConvUnroll], nxt[kConvUnroll];
#pragma unroll
        for (int u = 0; u < kConvUnroll; ++u)
            if (t0 + u < t1) cur[u] = IO::raw(xs, (int64_t)(t0 + u) * C + ch);
        for (int tb = t0; tb < t1; tb += kConvUnroll) {
            const int tn = tb + kConvUnroll;
#pragma unroll
            for (int u = 0; u < kConvUnroll; ++u)
                if (tn + u < t1) nxt[u] = IO::raw(xs, (int64_t)(tn + u) * C + ch);
#pragma unroll
            for (int u = 0; u < kConvUnroll; ++u) {
                if (tb + u < t1) {
                    float xv[kConvVec], o[kConvVec];
                    IO::unpack(cur[u], xv);
#pragma unroll
                    for (int v = 0; v < kConvVec; ++v) {
                        float z = bias[v];
#pragma unroll
                        for (int k = 0; k < W - 1; ++k) z = fmaf(w[k][v], win[k][v], z);
                        z = fmaf(w[W - 1][v], xv[v], z);
                        o[v] = a.silu ? silu(z) : z;
                    }
                    IO::store(os, (int64_t)(tb + u) * C + ch, o, true);
#pragma unroll
                    for (int i = 0; i + 1 < W - 1; ++i)
#pragma unroll
                        for (int v = 0; v < kConvVec; ++v) win[i][v] = win[i + 1][v];
                    if constexpr (W > 1) {
#pragma unroll
                        for (int v = 0; v < kConvVec; ++v) win[W - 2][v] = xv[v];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kConvUnroll; ++u) cur[u] = nxt[u];
        }
    }

    // the sequence's last W-1 inputs into its write slot
    if (last && ws >= 0) {
#pragma unroll
        for (int i = 0; i < W - 1; ++i) IO::store(a.states, ws * slot_elems + i * C + ch, win[i], false);
    }
}

template <typename T>
static hipError_t launch_conv1d_t(const Conv1dArgs &a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.channel_blocks * (a.max_chunks + a.S);
    const dim3 grid((unsigned)blocks), block(kConvThreads);
    switch (a.W) {
        case 1: hipLaunchKernelGGL((ssd_conv1d_kernel<T, 1>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((ssd_conv1d_kernel<T, 2>), grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL((ssd_conv1d_kernel<T, 3>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((ssd_conv1d_kernel<T, 4>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int32_t conv1d_channel_blocks(int32_t channels) {
    const int per = kConvThreads * kConvVec;
    return (channels + per - 1) / per;
}

hipError_t launch_conv1d(const Conv1dArgs &a, bool bf16, hipStream_t stream) {
    if ((int64_t)a.channel_blocks * (a.max_chunks + a.S) == 0) return hipSuccess;
    return bf16 ? launch_conv1d_t<__bf16>(a, stream) : launch_conv1d_t<float>(a, stream);
}

}  // namespace ssd
