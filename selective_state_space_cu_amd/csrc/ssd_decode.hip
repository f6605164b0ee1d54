// Decode step with dual state anchors: one new token per sequence advances the
// SSM state read from one cache slot and writes it to another (the read/write
// anchor split that the prefix-caching page gives the decode kernels, so that a
// block checkpoint is never overwritten by the running state).
//
// For sequence s, head h (group g = h / (H/G)):
//   S     = cache[read_slot[s], h]                 (zero if read_slot[s] < 0)
//   delta = softplus(dt[s,h] + dt_bias[h])
//   S'    = 2^(delta A[h] log2 e) S + delta x[s,h] B[s,g]^T
//   y     = S' C[s,g] + D[h] x[s,h]
//   cache[write_slot[s], h] = S'                   (skipped if write_slot[s] < 0)
//
// Memory-bound: the state slots are the traffic (2 x P x N x 4 bytes per
// (sequence, head)); x, B, C, dt and y are small. Each thread owns 4
// consecutive n of RPT state rows: 16-byte loads and stores, with N / 4 lanes
// covering one 512-byte row (N = 128) so that every wave-wide access is whole
// contiguous rows. All of a thread's state loads are issued before any math
// (RPT x 16 bytes in flight per lane). y[p] is a sum over the N / 4 lanes of
// row p (a butterfly over lane xor masks, inside the row's lane group).
#include "ssd_scan.hpp"

namespace ssd {

constexpr int kDecodeThreads = 128;   // measured: 128 / 256 / 512 threads -> 186.6 / 191.4 / 189.8 us
constexpr int kDecodeRowsPerThread = 2;   // 2: measured best of 1, 2, 4, 8 on the 256-sequence batch

template <typename T>
__device__ __forceinline__ float ld_f(const T *p) { return (float)*p; }

template <typename T, int N>
__global__ __launch_bounds__(kDecodeThreads) void ssd_decode_kernel(DecodeArgs a) {
    constexpr int LPR = N / 4;                       // lanes per state row
    constexpr int RPP = kDecodeThreads / LPR;        // rows per pass of the workgroup
    constexpr int RPT = kDecodeRowsPerThread;        // passes (rows per thread)
    static_assert(LPR >= 4 && LPR <= 64 && kDecodeThreads % LPR == 0, "dstate 16 .. 256");
    const int tid = threadIdx.x;
    const int nq = tid % LPR, rr = tid / LPR;
    const int H = a.H, P = a.P, G = a.G;

    int b = blockIdx.x;
    const int pc = b % a.pchunks;
    b /= a.pchunks;
    const int h = b % H, s = b / H;
    const int rs = a.read_slot[s], ws = a.write_slot[s];
    if (rs >= a.num_slots || ws >= a.num_slots) {   // refused: nothing read or written
        if (tid == 0 && pc == 0 && h == 0 && a.error_flag != nullptr) atomicOr(a.error_flag, SSD_DATA_BAD_SLOT);
        return;
    }
    const int g = h / (H / G);
    const int64_t slot_elems = (int64_t)H * P * N;
    const int64_t head_off = (int64_t)h * P * N + 4 * nq;
    const float *src = a.cache + (int64_t)(rs < 0 ? 0 : rs) * slot_elems + head_off;
    float *dst = a.cache + (int64_t)(ws < 0 ? 0 : ws) * slot_elems + head_off;
    const T *xs = reinterpret_cast<const T *>(a.x) + ((int64_t)s * H + h) * P;
    T *ys = reinterpret_cast<T *>(a.y) + ((int64_t)s * H + h) * P;
    const int p0 = pc * RPP * RPT + rr;

    // state rows first (the traffic), then the small operands
    f32x4 st[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int p = p0 + k * RPP;
        st[k] = (rs >= 0 && p < P)
                    ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + (int64_t)p * N))
                    : f32x4{0, 0, 0, 0};
    }
    float xv[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int p = p0 + k * RPP;
        xv[k] = p < P ? ld_f(xs + p) : 0.0f;
    }
    const T *Bs = reinterpret_cast<const T *>(a.B) + ((int64_t)s * G + g) * N + 4 * nq;
    const T *Cs = reinterpret_cast<const T *>(a.C) + ((int64_t)s * G + g) * N + 4 * nq;
    float bv[4], cv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        bv[j] = ld_f(Bs + j);
        cv[j] = ld_f(Cs + j);
    }
    const float delta = softplus_hw(a.dt[(int64_t)s * H + h] + (a.dt_bias ? a.dt_bias[h] : 0.0f));
    const float decay = fast_exp2(delta * a.A[h] * kLog2e);
    const float Dh = a.D ? a.D[h] : 0.0f;

#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int p = p0 + k * RPP;
        const float dx = delta * xv[k];
        f32x4 o;
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[j] = fmaf(decay, st[k][j], dx * bv[j]);
            part = fmaf(cv[j], o[j], part);
        }
        if (ws >= 0 && p < P) __builtin_nontemporal_store(o, reinterpret_cast<f32x4 *>(dst + (int64_t)p * N));
        // sum over the row's LPR lanes (all lanes take part; lane groups are aligned)
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, LPR);
        if (nq == 0 && p < P) ys[p] = (T)(part + Dh * xv[k]);
    }
}

template <typename T>
static hipError_t launch_decode_t(const DecodeArgs &a, int dstate, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.S * a.H * a.pchunks;
    const dim3 grid((unsigned)blocks), block(kDecodeThreads);
    switch (dstate) {
        case 16: hipLaunchKernelGGL((ssd_decode_kernel<T, 16>), grid, block, 0, stream, a); break;
        case 32: hipLaunchKernelGGL((ssd_decode_kernel<T, 32>), grid, block, 0, stream, a); break;
        case 64: hipLaunchKernelGGL((ssd_decode_kernel<T, 64>), grid, block, 0, stream, a); break;
        case 128: hipLaunchKernelGGL((ssd_decode_kernel<T, 128>), grid, block, 0, stream, a); break;
        case 256: hipLaunchKernelGGL((ssd_decode_kernel<T, 256>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int32_t decode_pchunks(int32_t headdim, int32_t dstate) {
    const int rows_per_block = kDecodeThreads / (dstate / 4) * kDecodeRowsPerThread;
    return (headdim + rows_per_block - 1) / rows_per_block;
}

hipError_t launch_decode(const DecodeArgs &a, bool bf16, int dstate, hipStream_t stream) {
    if ((int64_t)a.S * a.H * a.pchunks == 0) return hipSuccess;
    return bf16 ? launch_decode_t<__bf16>(a, dstate, stream) : launch_decode_t<float>(a, dstate, stream);
}

}  // namespace ssd
