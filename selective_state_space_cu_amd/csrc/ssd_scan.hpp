// Fused chunk-walk kernel of the Mamba2 SSD varlen scan for gfx950.
//
// One workgroup owns one (sequence, head, headdim tile of 16*NW columns) and
// walks that sequence's chunks in order; each of its NW waves owns 16 headdim
// columns and carries their (16 x N) float32 state in registers from chunk to
// chunk, so chunk states never round-trip through HBM (only exported
// checkpoints and final states are written).
//
// Per chunk (the chunked decomposition of the SSD layer; the numbers follow the
// kernel list of the problem statement):
//   (2) delta_j = softplus(dt_j + dt_bias), cumulative log-decay s_j =
//       sum_{k<=j} delta_k*A (inclusive, chunk-local, log2 units), plus the
//       per-token factors 2^(s_i) and w_j = delta_j 2^(s_last - s_j), one wave,
//       one chunk ahead of its use;
//   (5) CB^T = B . C^T per 16x16 sub-tile on the matrix cores, masked by the
//       segment-sum decay: M[i][j] = CB[i][j] * 2^(s_i - s_j) * delta_j, j <= i;
//   (6) Y^T = h_in . C^T scaled per token by 2^(s_i)   (inter-chunk term)
//           + x^T . M^T                                (intra-chunk term)
//           + D x;
//   (3,4) h_out = 2^(s_last) h_in + B^T . (w o x).
// The decay that reaches the entering state at token i is 2^(s_i) with s_i
// the INCLUSIVE cumsum at i, and the chunk's total decay is read at the chunk's
// last valid token -- never at a tile start or past the sequence end (the
// init-state decay rule of the varlen bug-fix page).
//
// Chunks longer than 64 tokens run as 64-row M-tiles; M-tile m streams the
// chunk's K-tiles 0..m (quadratic intra-chunk form over the whole chunk), and
// the last M-tile also accumulates the chunk state. A "step" is one
// (chunk, M-tile, K-tile) triple.
//
// Memory pipeline: the B, C and x tiles (and the next chunk's dt) of step
// i + NST - 1 are fetched with direct-to-LDS buffer loads while step i
// computes (NST stage buffers). Every step issues the same number of vector
// memory instructions (out-of-range buffer lanes are zero-filled on load and
// dropped on store), so an exact s_waitcnt vmcnt(n) waits for one stage only;
// barriers are bare s_barrier after an LDS-count wait. Tile rows in LDS are
// padded by 16 bytes, which keeps the row-strided and transposed fragment reads
// below free of bank conflicts and their addresses affine (a per-lane base plus
// compile-time offsets); the direct loads skip the pad slots.
//
// Operand layouts on the matrix cores (v_mfma_f32_16x16x32_bf16; the f32 path
// issues eight v_mfma_f32_16x16x4f32 per 32-deep step with the same
// fragments): lane l = 16*g + q supplies row/column q and the 8 "k slots" of
// group g. Any assignment of k indices to (g, slot) is valid as long as both
// operands use the same one, which lets
//   - token-major tiles in LDS feed operands that contract over tokens through
//     the gfx950 LDS transpose read (ds_read_b64_tr_b16), and
//   - the carried state, held in the accumulator layout of B^T.(w o x), feed the
//     inter-chunk product directly from registers (C is read with the matching
//     permuted k order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_internal.h"

namespace ssd {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTile = 64;       // tokens per M-/K-tile
constexpr int kMaxChunk = 256;  // largest supported chunk_size
constexpr int kLdsLimit = 160 * 1024;
constexpr int kBufFlags = 0x00020000;  // raw buffer resource word 3 on gfx9-family parts
constexpr int kOob = 0x40000000;       // buffer offset beyond every tile's range (zero fill / dropped)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

__device__ __forceinline__ float softplus(float u) { return u > 20.0f ? u : log1pf(expf(u)); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int VM> struct WaitVm {
    static_assert(VM >= 0 && VM <= 63, "vmcnt out of range");
    static constexpr int imm = (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8);
};
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Workgroup barrier for LDS data: waits for this wave's LDS operations only
// (vector memory, including direct-to-LDS loads in flight, is waited for
// explicitly). The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)(p);
}
__device__ __forceinline__ const unsigned char *lds_ptr(uint32_t a) {
    return (const unsigned char *)(const __attribute__((address_space(3))) unsigned char *)(uintptr_t)a;
}

// ---------------------------------------------------------------------------
// Element traits: fragment type, LDS tile reads, matrix op. A tile row holds
// `pitch` bytes (data + 16 bytes of padding); element e of row r is at
// r*pitch + e*sizeof(T).
// ---------------------------------------------------------------------------
template <typename T> struct Ops;

template <typename T>
__device__ __forceinline__ int lds_off(int row, int e, int pitch) { return row * pitch + e * (int)sizeof(T); }

// bfloat16 (stored as uint16_t)
template <> struct Ops<uint16_t> {
    struct Frag { u32x4 w; };
    static constexpr int kPad = 8;  // decay matrix row padding (elements)

    __device__ static f32x4 mma(f32x4 acc, const Frag &a, const Frag &b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.w),
                                                       __builtin_bit_cast(bf16x8, b.w), acc, 0, 0, 0);
    }
    // slots s <- tile[row][k + s] (k a multiple of 8)
    __device__ static Frag rowk(const unsigned char *t, int pitch, int row, int k) {
        return Frag{*reinterpret_cast<const u32x4 *>(t + lds_off<uint16_t>(row, k, pitch))};
    }
    // slots 0..3 <- tile[row][k0 + 4g + s]; slots 4..7 <- tile[row][k0 + 16 + 4g + s - 4]
    __device__ static Frag rowk_perm(const unsigned char *t, int pitch, int row, int k0, int g) {
        u32x2 lo = *reinterpret_cast<const u32x2 *>(t + lds_off<uint16_t>(row, k0 + 4 * g, pitch));
        u32x2 hi = *reinterpret_cast<const u32x2 *>(t + lds_off<uint16_t>(row, k0 + 16 + 4 * g, pitch));
        return Frag{u32x4{lo.x, lo.y, hi.x, hi.y}};
    }
    // Transposed fragment reads of a token-major tile: slots s <- tile[kb + s][col0 + q].
    // Within each 16-lane group, lane q supplies the 4 elements at row kb + q/4,
    // columns col0 + 4(q%4)..+3, and receives column col0 + q of rows kb..kb+3
    // (ds_read_b64_tr_b16; a fragment is two reads, rows kb.. and kb+4..).
    // `addr` is this lane's LDS byte address for the first fragment; fragment f
    // is at byte offset F_f (a compile-time immediate). The reads are issued as
    // one inline-asm statement that also waits for them, so in-flight
    // direct-to-LDS loads are not drained and no register holds a pending value
    // outside the statement.
    __device__ static uint32_t tr_addr(const unsigned char *t, int pitch, int kb, int col0, int q) {
        return lds_addr(t + (kb + (q >> 2)) * pitch + (col0 + 4 * (q & 3)) * 2);
    }
    // Same, but the fragment's 16 columns are the paired-state rows
    // {8m + j : m, j = 0..3} (+ the tile's immediate offset): source lane q
    // supplies the 4 columns at 8 (q%4), so result lane q gets column 8 (q/4) + q%4.
    __device__ static uint32_t tr_addr_pairs(const unsigned char *t, int pitch, int kb, int q) {
        return lds_addr(t + (kb + (q >> 2)) * pitch + 8 * (q & 3) * 2);
    }
    template <int F0, int F1, int R4>   // R4 = 4 * pitch (second read of a fragment)
    __device__ static void tr2(uint32_t addr, Frag &a, Frag &b) {
        u32x2 r0, r1, r2, r3;
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4 offset:%5\n\t"
            "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
            "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
            "ds_read_b64_tr_b16 %3, %4 offset:%8\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
            : "v"(addr), "i"(F0), "i"(F0 + R4), "i"(F1), "i"(F1 + R4));
        a = Frag{u32x4{r0.x, r0.y, r1.x, r1.y}};
        b = Frag{u32x4{r2.x, r2.y, r3.x, r3.y}};
    }
    template <int F0, int F1, int F2, int F3, int R4>
    __device__ static void tr4(uint32_t addr, Frag &a, Frag &b, Frag &c, Frag &d) {
        u32x2 r0, r1, r2, r3, r4, r5, r6, r7;
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8 offset:%9\n\t"
            "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
            "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
            "ds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
            "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
            "ds_read_b64_tr_b16 %5, %8 offset:%14\n\t"
            "ds_read_b64_tr_b16 %6, %8 offset:%15\n\t"
            "ds_read_b64_tr_b16 %7, %8 offset:%16\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
            : "v"(addr), "i"(F0), "i"(F0 + R4), "i"(F1), "i"(F1 + R4), "i"(F2), "i"(F2 + R4), "i"(F3),
              "i"(F3 + R4));
        a = Frag{u32x4{r0.x, r0.y, r1.x, r1.y}};
        b = Frag{u32x4{r2.x, r2.y, r3.x, r3.y}};
        c = Frag{u32x4{r4.x, r4.y, r5.x, r5.y}};
        d = Frag{u32x4{r6.x, r6.y, r7.x, r7.y}};
    }
    __device__ static void load4(const unsigned char *t, int pitch, int row, int e, float (&v)[4]) {
        u32x2 w = *reinterpret_cast<const u32x2 *>(t + lds_off<uint16_t>(row, e, pitch));
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    }
    // decay matrix (padded row-major, not swizzled)
    __device__ static Frag mrow(const uint16_t *m, int pitch, int row, int k) {
        return Frag{*reinterpret_cast<const u32x4 *>(m + row * pitch + k)};
    }
    __device__ static void mstore4(uint16_t *m, int pitch, int row, int col, const float (&v)[4]) {
        *reinterpret_cast<u32x2 *>(m + row * pitch + col) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    }
    __device__ static Frag from_f32(const f32x4 &lo, const f32x4 &hi) {
        return Frag{u32x4{pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]), pack_bf16(hi[0], hi[1]),
                          pack_bf16(hi[2], hi[3])}};
    }
    __device__ static Frag low_half(const Frag &f) { return Frag{u32x4{f.w[0], f.w[1], 0u, 0u}}; }
    __device__ static Frag scale(const Frag &f, const float (&w)[8]) {
        Frag r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.w[i] = pack_bf16(bf16_lo(f.w[i]) * w[2 * i], bf16_hi(f.w[i]) * w[2 * i + 1]);
        return r;
    }
    // 4 output values (consecutive headdim columns) -> y
    __device__ static void store_y(__amdgpu_buffer_rsrc_t r, int off, const float (&v)[4]) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, r, off, 0, 0);
    }
};

// float32
template <> struct Ops<float> {
    struct Frag { float v[8]; };
    static constexpr int kPad = 4;

    __device__ static f32x4 mma(f32x4 acc, const Frag &a, const Frag &b) {
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
        return acc;
    }
    __device__ static Frag rowk(const unsigned char *t, int pitch, int row, int k) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(t + lds_off<float>(row, k, pitch));
        f32x4 b = *reinterpret_cast<const f32x4 *>(t + lds_off<float>(row, k + 4, pitch));
        return Frag{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
    }
    __device__ static Frag rowk_perm(const unsigned char *t, int pitch, int row, int k0, int g) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(t + lds_off<float>(row, k0 + 4 * g, pitch));
        f32x4 b = *reinterpret_cast<const f32x4 *>(t + lds_off<float>(row, k0 + 16 + 4 * g, pitch));
        return Frag{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
    }
    __device__ static uint32_t tr_addr(const unsigned char *t, int pitch, int kb, int col0, int q) {
        return lds_addr(t + kb * pitch + (col0 + q) * 4);
    }
    __device__ static uint32_t tr_addr_pairs(const unsigned char *t, int pitch, int kb, int q) {
        return lds_addr(t + kb * pitch + (8 * (q >> 2) + (q & 3)) * 4);
    }
    __device__ static Frag tr_one(uint32_t addr, int pitch) {
        const unsigned char *p = lds_ptr(addr);
        Frag f;
#pragma unroll
        for (int s = 0; s < 8; ++s) f.v[s] = *reinterpret_cast<const float *>(p + s * pitch);
        return f;
    }
    template <int F0, int F1, int R4>
    __device__ static void tr2(uint32_t addr, Frag &a, Frag &b) {
        a = tr_one(addr + F0, R4 / 4);
        b = tr_one(addr + F1, R4 / 4);
    }
    template <int F0, int F1, int F2, int F3, int R4>
    __device__ static void tr4(uint32_t addr, Frag &a, Frag &b, Frag &c, Frag &d) {
        a = tr_one(addr + F0, R4 / 4);
        b = tr_one(addr + F1, R4 / 4);
        c = tr_one(addr + F2, R4 / 4);
        d = tr_one(addr + F3, R4 / 4);
    }
    __device__ static void load4(const unsigned char *t, int pitch, int row, int e, float (&v)[4]) {
        f32x4 w = *reinterpret_cast<const f32x4 *>(t + lds_off<float>(row, e, pitch));
        v[0] = w[0]; v[1] = w[1]; v[2] = w[2]; v[3] = w[3];
    }
    __device__ static Frag mrow(const float *m, int pitch, int row, int k) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(m + row * pitch + k);
        f32x4 a = p[0], b = p[1];
        return Frag{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
    }
    __device__ static void mstore4(float *m, int pitch, int row, int col, const float (&v)[4]) {
        *reinterpret_cast<f32x4 *>(m + row * pitch + col) = f32x4{v[0], v[1], v[2], v[3]};
    }
    __device__ static Frag from_f32(const f32x4 &lo, const f32x4 &hi) {
        return Frag{{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}};
    }
    __device__ static Frag low_half(const Frag &f) { return Frag{{f.v[0], f.v[1], f.v[2], f.v[3], 0, 0, 0, 0}}; }
    __device__ static Frag scale(const Frag &f, const float (&w)[8]) {
        Frag r;
#pragma unroll
        for (int s = 0; s < 8; ++s) r.v[s] = f.v[s] * w[s];
        return r;
    }
    __device__ static void store_y(__amdgpu_buffer_rsrc_t r, int off, const float (&v)[4]) {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                     __float_as_uint(v[2]), __float_as_uint(v[3])},
                                               r, off, 0, 0);
    }
};

template <typename T, int NW, int N>
struct ScanShape {
    static constexpr int kThreads = 64 * NW;
    static constexpr int kCols = 16 * NW;            // headdim columns per workgroup
    static constexpr int kES = sizeof(T);
    static constexpr int kNE = N < 32 ? 32 : N;      // state width in LDS / registers (zero-padded)
    static constexpr int kRG = N * kES;              // bytes per B/C row in global memory
    static constexpr int kRB = kNE * kES;            // data bytes per B/C tile row in LDS
    static constexpr int kRX = kCols * kES;          // data bytes per x tile row
    static constexpr int kPB = kRB + 16;             // padded LDS row pitch (B/C)
    static constexpr int kPX = kRX + 16;             // padded LDS row pitch (x)
    static constexpr int kTileB = kTile * kPB;       // a multiple of 1 KB
    static constexpr int kTileX = kTile * kPX;
    static constexpr int kIB = (kTileB / 1024 + NW - 1) / NW;   // 1 KB load instructions per wave (B, and C)
    static constexpr int kIX = (kTileX / 1024 + NW - 1) / NW;   // (x)
    static constexpr int kID = (4 + NW - 1) / NW;               // (dt: 4 x 64 floats)
    static constexpr int kLoads = 2 * kIB + kIX + kID;          // vector memory loads per wave per step
    static constexpr int kNT = kNE / 16;                        // 16-row state tiles (even)
    static constexpr int kYStores = 4;                          // y stores per wave per step
    static constexpr int kNK = kNE / 32;                        // 32-deep steps over dstate
    static constexpr int kMP = kTile + Ops<T>::kPad;            // decay matrix pitch (elements)
    // LDS: NST stages of [B | C | x | dt(256 f32)] + decay matrix + 2 scan tables + 1 KB sink
    static constexpr int kStage = 2 * kTileB + kTileX + 1024;
    static constexpr int kFixed = kTile * kMP * kES + 2 * 4 * kMaxChunk * 4 + 1024;
    static constexpr int fit(int n) { return n * kStage + kFixed <= kLdsLimit; }
    // vector memory instructions a wave issued after the loads of the stage it
    // waits for: the later stages' loads, and the stores of the steps since
    // (4 y stores each, plus kNT state stores per step that exported a checkpoint)
    static constexpr int vm_wait(int n, int exports) {
        return (n - 2) * kLoads + (n - 1) * kYStores + exports * kNT;
    }
    static constexpr int pick() {
        return (fit(3) && vm_wait(3, 2) <= 63) ? 3 : ((fit(2) && vm_wait(2, 1) <= 63) ? 2 : 1);
    }
    static constexpr int kNST = pick();
    static constexpr int kLdsBytes = kNST * kStage + kFixed;
    static_assert(fit(1), "tile does not fit in LDS");
};

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then row
// broadcasts across the four 16-lane rows).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_scan(float v) {
    v += dpp_mov<0x111, 0xf>(v);   // row_shr:1
    v += dpp_mov<0x112, 0xf>(v);   // row_shr:2
    v += dpp_mov<0x114, 0xf>(v);   // row_shr:4
    v += dpp_mov<0x118, 0xf>(v);   // row_shr:8
    v += dpp_mov<0x142, 0xa>(v);   // row_bcast:15 -> rows 1, 3
    v += dpp_mov<0x143, 0xc>(v);   // row_bcast:31 -> rows 2, 3
    return v;
}

// softplus(u) = max(u, 0) + ln(1 + e^-|u|), on the hardware exp2/log2
__device__ __forceinline__ float softplus_hw(float u) {
    const float z = fast_exp2(-fabsf(u) * kLog2e);
    return fmaxf(u, 0.0f) + __builtin_amdgcn_logf(1.0f + z) * 0.6931471805599453f;
}

// Per-chunk scan tables (log2-unit cumsum, delta, 2^s_i, w_j), one wave.
// raw(j) returns dt of token j (j < Lc).
template <typename RawDt>
__device__ __forceinline__ void chunk_scan(float *tab, int Lc, float bias, float a2, int lane, RawDt raw) {
    float *sS = tab, *sD = tab + kMaxChunk, *sE = tab + 2 * kMaxChunk, *sW = tab + 3 * kMaxChunk;
    float v_keep[kMaxChunk / 64], d_keep[kMaxChunk / 64];
    float carry = 0.0f;
#pragma unroll
    for (int piece = 0; piece < kMaxChunk / 64; ++piece) {
        const int j = piece * 64 + lane;
        float d = 0.0f, v = 0.0f;
        if (piece * 64 < Lc) {
            if (j < Lc) {
                d = softplus_hw(raw(j) + bias);
                v = d * a2;
            }
            v = wave_scan(v) + carry;
            carry = __shfl(v, 63, 64);
        }
        v_keep[piece] = v;
        d_keep[piece] = d;
    }
    const float sL = carry;   // cumsum at the chunk's last valid token (invalid tokens add 0)
#pragma unroll
    for (int piece = 0; piece < kMaxChunk / 64; ++piece) {
        if (piece * 64 < Lc) {
            const int j = piece * 64 + lane;
            const float v = v_keep[piece], d = d_keep[piece];
            sS[j] = v;
            sD[j] = d;
            sE[j] = fast_exp2(v);
            sW[j] = j < Lc ? d * fast_exp2(sL - v) : 0.0f;
        }
    }
}

// Transposed reads of the NT state-tile fragments of B^T (rows n of the paired
// state layout) sharing one base address (tr_addr_pairs): tile t = 2c + u
// starts at column 32 c + 4 u.
template <typename O, int NT, int ES, int R4, int T0 = 0>
__device__ __forceinline__ void tr_tiles(uint32_t addr, typename O::Frag (&f)[NT]) {
    constexpr auto off = [](int t) { return (32 * (t >> 1) + 4 * (t & 1)) * ES; };
    if constexpr (T0 + 4 <= NT) {
        O::template tr4<off(T0), off(T0 + 1), off(T0 + 2), off(T0 + 3), R4>(addr, f[T0], f[T0 + 1], f[T0 + 2],
                                                                            f[T0 + 3]);
        tr_tiles<O, NT, ES, R4, T0 + 4>(addr, f);
    } else if constexpr (T0 + 2 <= NT) {
        O::template tr2<off(T0), off(T0 + 1), R4>(addr, f[T0], f[T0 + 1]);
        tr_tiles<O, NT, ES, R4, T0 + 2>(addr, f);
    }
}

// One workgroup per CU (the stage buffers take most of the LDS), i.e. one wave
// per SIMD: let the scheduler spend registers on hoisting LDS reads ahead of
// the matrix ops instead of targeting an occupancy the LDS cannot give.
template <typename T, int NW, int N>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ssd_scan_kernel(ScanArgs a, const int32_t *__restrict__ dstmap)
#if !defined(__HIP_DEVICE_COMPILE__)
{   // the host pass only needs the signature (for the launch stub)
}
#else
{
    using O = Ops<T>;
    using Frag = typename O::Frag;
    using SH = ScanShape<T, NW, N>;
    constexpr int NST = SH::kNST, RG = SH::kRG, RX = SH::kRX, PB = SH::kPB, PX = SH::kPX;
    constexpr int MP = SH::kMP, ES = SH::kES, NT = SH::kNT, NK = SH::kNK;
    constexpr int JS = (4 + NW - 1) / NW;   // decay-matrix column blocks per wave

    extern __shared__ __align__(16) unsigned char smem[];
    T *sM = reinterpret_cast<T *>(smem + NST * SH::kStage);                              // [kTile][MP]
    float *tabs = reinterpret_cast<float *>(smem + NST * SH::kStage + kTile * MP * ES);  // 2 x [4][kMaxChunk]
    unsigned char *sink = smem + NST * SH::kStage + kTile * MP * ES + 2 * 4 * kMaxChunk * 4;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (kept in an SGPR)
    const int q = lane & 15, g = lane >> 4;

    if (__builtin_nontemporal_load(a.error_flag) & SSD_DATA_BAD_CU_SEQLENS) return;
    const int per_seq = a.H * a.nptiles;
    const int rank = blockIdx.x / per_seq;
    const int rem = blockIdx.x - rank * per_seq;
    const int h = rem / a.nptiles, pt = rem - h * a.nptiles;
    const int s = a.seq_order[rank];
    if (s < 0 || s >= a.S) return;
    const int grp = h / (a.H / a.G);
    const int H = a.H, P = a.P, G = a.G, cs = a.cs;
    int64_t tb = a.cu_seqlens[s], te = a.cu_seqlens[s + 1];
    tb = tb < 0 ? 0 : (tb > a.T ? a.T : tb);
    te = te < tb ? tb : (te > a.T ? a.T : te);
    const int L = (int)(te - tb);
    const int nch = (L + cs - 1) / cs;
    const int c0 = a.seq_chunk_start[s];
    const int p0 = pt * SH::kCols;       // first headdim column of the workgroup
    const int pw = p0 + 16 * wave;       // first headdim column of this wave
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float a2 = a.A[h] * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const T *xg = reinterpret_cast<const T *>(a.x);
    const T *Bg = reinterpret_cast<const T *>(a.B);
    const T *Cg = reinterpret_cast<const T *>(a.C);
    T *yg = reinterpret_cast<T *>(a.y);
    const int scan_wave = NW - 1;
    const int xrow = H * P * ES;    // bytes between tokens of x / y
    const int brow = G * N * ES;    // bytes between tokens of B / C

    auto chunk_len = [&](int k) { return min(cs, L - k * cs); };
    auto ntiles = [&](int k) { return (chunk_len(k) + kTile - 1) / kTile; };
    // step order: chunk k, M-tile m, K-tile kt = 0..m
    auto advance = [&](int &k, int &m, int &kt) {
        if (++kt > m) { kt = 0; if (++m >= ntiles(k)) { m = 0; ++k; } }
    };

    // Carried state, in pairs of 16-row tiles: st[2c+u][r] = h[p = pw + q][n = 32 c + 8 g + 4 u + r],
    // i.e. lane group g holds the 8 consecutive n that the 32-deep operand slots of
    // group g cover, so the state feeds C . h^T with the same C fragments as C . B^T.
    // Rows n >= N (dstate < 32 only) stay zero.
    f32x4 st[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) st[t] = f32x4{0, 0, 0, 0};
    auto state_n = [&](int t) { return 32 * (t >> 1) + 8 * g + 4 * (t & 1); };
    if (a.init != nullptr && (a.has_init == nullptr || a.has_init[s] != 0)) {
        const float *src = a.init + ((int64_t)(s * H + h) * P + pw + q) * N;
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (state_n(t) < N) st[t] = *reinterpret_cast<const f32x4 *>(src + state_n(t));
    }

    // scan tables of chunk 0, from global dt
    if (nch > 0 && wave == scan_wave) {
        const float *dt0 = a.dt + tb * H + h;
        chunk_scan(tabs, chunk_len(0), bias, a2, lane, [&](int j) { return dt0[(int64_t)j * H]; });
    }
    __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);   // nothing outstanding before the tile pipeline starts

    // Per-lane parts of the direct-to-LDS loads (loop invariant). Lane l of load
    // block j fills LDS bytes [1024 j + 16 l, +16) of a tile: row r = that / pitch;
    // bytes of the row padding get an out-of-range offset (zero fill).
    struct GlobalOffsets { int b[SH::kIB], x[SH::kIX], d[SH::kID]; } go;
#pragma unroll
    for (int i = 0; i < SH::kIB; ++i) {
        const int j = wave + NW * i, o = 1024 * j + 16 * lane, r = o / PB, pos = o % PB;
        go.b[i] = (j < SH::kTileB / 1024 && pos < RG) ? r * brow + pos : kOob;
    }
#pragma unroll
    for (int i = 0; i < SH::kIX; ++i) {
        const int j = wave + NW * i, o = 1024 * j + 16 * lane, r = o / PX, pos = o % PX;
        go.x[i] = (j < SH::kTileX / 1024 && pos < RX) ? r * xrow + pos : kOob;
    }
#pragma unroll
    for (int i = 0; i < SH::kID; ++i) {
        const int j = wave + NW * i;
        go.d[i] = j < 4 ? (64 * j + lane) * H * 4 : kOob;
    }

    // Fetch the tiles of step (k, m, kt) into stage buffer `slot` (out-of-range,
    // zero-filling loads when k >= nch), in two parts issued at different points
    // of a step. Always 2*kIB + kIX + kID instructions per wave.
    auto fetch_bc = [&](int slot, int k, int m, int kt) {
        unsigned char *stg = smem + slot * SH::kStage;
        const bool live = k < nch;
        const int Lc = live ? chunk_len(k) : 0;
        const int64_t t0 = tb + (int64_t)k * cs;
        const int vk = live ? min(kTile, Lc - kTile * kt) : 0;
        const int vm = live ? min(kTile, Lc - kTile * m) : 0;
        const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Bg + ((t0 + kTile * kt) * G + grp) * N), 0, vk * brow, kBufFlags);
        const __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Cg + ((t0 + kTile * m) * G + grp) * N), 0, vm * brow, kBufFlags);
#pragma unroll
        for (int i = 0; i < SH::kIB; ++i) {
            const int j = wave + NW * i;   // 1 KB block of the tile
            const bool ok = j < SH::kTileB / 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void *)(ok ? stg + 1024 * j : sink), 16, go.b[i], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rC, (lds_void *)(ok ? stg + SH::kTileB + 1024 * j : sink), 16,
                                                     go.b[i], 0, 0, 0);
        }
    };
    auto fetch_xd = [&](int slot, int k, int m, int kt) {
        unsigned char *stg = smem + slot * SH::kStage;
        const bool live = k < nch;
        const int Lc = live ? chunk_len(k) : 0;
        const int64_t t0 = tb + (int64_t)k * cs;
        const int vk = live ? min(kTile, Lc - kTile * kt) : 0;
        const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(xg + ((t0 + kTile * kt) * H + h) * P + p0), 0, vk * xrow, kBufFlags);
        // dt of chunk k+1 rides with the first step of chunk k
        const bool dnext = live && m == 0 && kt == 0 && k + 1 < nch;
        const int64_t t1 = tb + (int64_t)(k + 1) * cs;
        const __amdgpu_buffer_rsrc_t rD = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.dt + (dnext ? t1 : 0) * H + h), 0, dnext ? chunk_len(k + 1) * H * 4 : 0, kBufFlags);
#pragma unroll
        for (int i = 0; i < SH::kIX; ++i) {
            const int j = wave + NW * i;
            const bool ok = j < SH::kTileX / 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, (lds_void *)(ok ? stg + 2 * SH::kTileB + 1024 * j : sink), 16,
                                                     go.x[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < SH::kID; ++i) {
            const int j = wave + NW * i;   // 64-token block of dt
            const bool ok = j < 4;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rD, (lds_void *)(ok ? stg + 2 * SH::kTileB + SH::kTileX + 256 * j : sink), 4, go.d[i], 0, 0, 0);
        }
    };
    // y stores of a step that writes no y (keeps the per-step count fixed)
    const __amdgpu_buffer_rsrc_t r_none = __builtin_amdgcn_make_buffer_rsrc((void *)yg, 0, 0, kBufFlags);
    auto dummy_y_stores = [&]() {
        const float z[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < SH::kYStores; ++i) O::store_y(r_none, 0, z);
    };
    auto wait_stage = [&](int exports) {   // exports among the last NST-1 steps
        if constexpr (NST == 3) {
            if (exports == 0) __builtin_amdgcn_s_waitcnt(WaitVm<SH::vm_wait(3, 0)>::imm);
            else if (exports == 1) __builtin_amdgcn_s_waitcnt(WaitVm<SH::vm_wait(3, 1)>::imm);
            else __builtin_amdgcn_s_waitcnt(WaitVm<SH::vm_wait(3, 2)>::imm);
        } else if constexpr (NST == 2) {
            if (exports == 0) __builtin_amdgcn_s_waitcnt(WaitVm<SH::vm_wait(2, 0)>::imm);
            else __builtin_amdgcn_s_waitcnt(WaitVm<SH::vm_wait(2, 1)>::imm);
        }
    };

    // prologue: stages of steps 0 .. NST-2
    int fk = 0, fm = 0, fkt = 0;   // fetch cursor
    if constexpr (NST > 1) {
#pragma unroll
        for (int p = 0; p < NST - 1; ++p) {
            fetch_bc(p, fk, fm, fkt);
            fetch_xd(p, fk, fm, fkt);
            if (fk < nch) advance(fk, fm, fkt);
            dummy_y_stores();
        }
    }

    f32x4 acc[4];  // Y^T tile: acc[it][r] = y[i = 16 it + q][p = pw + 4 g + r]
    int k = 0, m = 0, kt = 0;
    int ex1 = 0, ex2 = 0;   // did the previous / second previous step export a state
    for (int step = 0; k < nch; ++step) {
        const int slot = step % NST;
        const unsigned char *stg = smem + slot * SH::kStage;
        const unsigned char *sB = stg, *sC = stg + SH::kTileB, *sX = stg + 2 * SH::kTileB;
        const float *sDt = reinterpret_cast<const float *>(stg + 2 * SH::kTileB + SH::kTileX);
        const float *tab = tabs + (k & 1) * 4 * kMaxChunk;
        const float *sS = tab, *sD = tab + kMaxChunk, *sE = tab + 2 * kMaxChunk, *sW = tab + 3 * kMaxChunk;
        const int64_t t0 = tb + (int64_t)k * cs;
        const int Lc = chunk_len(k);
        const int ntile = (Lc + kTile - 1) / kTile;
        const bool last_m = (m == ntile - 1);

        if constexpr (NST == 1) {
            fetch_bc(0, k, m, kt);
            fetch_xd(0, k, m, kt);
            __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);
        } else {
            wait_stage(NST == 3 ? ex1 + ex2 : ex1);
        }
        lds_barrier();   // stage `slot` and this chunk's scan tables are visible
        // checkpoint slot of this chunk (scalar load, consumed at the chunk's end)
        int dst = -1;
        if (a.chunk_states != nullptr && last_m && kt == m) {
            const int gc = c0 + k;
            if (gc >= 0 && gc < a.max_chunks) dst = dstmap ? dstmap[gc] : gc;
        }
        if (m == 0 && kt == 0 && k + 1 < nch && wave == scan_wave) {
            // scan tables of the next chunk, from the dt that rode with this stage
            chunk_scan(tabs + ((k + 1) & 1) * 4 * kMaxChunk, chunk_len(k + 1), bias, a2, lane,
                       [&](int j) { return sDt[j]; });
        }
        const float sL = sS[Lc - 1];   // chunk total decay, at its last valid token

        // C fragments of M-tile m (rows i; 32-deep slots n = 32 c + 8 g + s), shared by
        // the inter-chunk product and C . B^T, and B fragments of this wave's
        // column blocks jsub = wave + NW*jj
        Frag cfm[4][NK], bf[JS][NK];
        float ei[4], si[4], sj[JS][4], dj[JS][4];
#pragma unroll
        for (int isub = 0; isub < 4; ++isub) {
#pragma unroll
            for (int c = 0; c < NK; ++c) cfm[isub][c] = O::rowk(sC, PB, 16 * isub + q, 32 * c + 8 * g);
            si[isub] = sS[kTile * m + 16 * isub + q];
            ei[isub] = sE[kTile * m + 16 * isub + q];
        }
#pragma unroll
        for (int jj = 0; jj < JS; ++jj) {
            const int jsub = (wave + NW * jj) & 3;
#pragma unroll
            for (int c = 0; c < NK; ++c) bf[jj][c] = O::rowk(sB, PB, 16 * jsub + q, 32 * c + 8 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int jc = kTile * kt + 16 * jsub + 4 * g + r;
                sj[jj][r] = sS[jc];
                dj[jj][r] = sD[jc];
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        if (kt == 0) {
            // (6) inter-chunk term Y^T = h_in . C^T, then scale column i by 2^(s_i)
#pragma unroll
            for (int it = 0; it < 4; ++it) acc[it] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < NK; ++c) {
                const Frag hf = O::from_f32(st[2 * c], st[2 * c + 1]);
#pragma unroll
                for (int it = 0; it < 4; ++it) acc[it] = O::mma(acc[it], hf, cfm[it][c]);
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) acc[it] *= ei[it];
            if (last_m) {
                // (4) the entering state decays over the whole chunk
                const float e = fast_exp2(sL);
#pragma unroll
                for (int t = 0; t < NT; ++t) st[t] *= e;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NST > 1) fetch_bc((step + NST - 1) % NST, fk, fm, fkt);   // overlaps the matrix ops

        // (5) CB^T sub-tiles of (M-tile m, K-tile kt) -> masked decay matrix in LDS;
        // sub-tiles above the diagonal come out as zeros through the mask
#pragma unroll
        for (int jj = 0; jj < JS; ++jj) {
            const int jsub = (wave + NW * jj) & 3;
            if (wave + NW * jj < 4) {
#pragma unroll
                for (int isub = 0; isub < 4; ++isub) {
                    f32x4 cb = {0, 0, 0, 0};
#pragma unroll
                    for (int c = 0; c < NK; ++c) cb = O::mma(cb, bf[jj][c], cfm[isub][c]);
                    const int il = 16 * isub + q, ic = kTile * m + il;
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int jc = kTile * kt + 16 * jsub + 4 * g + r;
                        const float dec = fast_exp2(si[isub] - sj[jj][r]) * dj[jj][r];
                        v[r] = (jc <= ic && ic < Lc) ? cb[r] * dec : 0.0f;
                    }
                    O::mstore4(sM, MP, il, 16 * jsub + 4 * g, v);
                }
            }
        }
        lds_barrier();   // decay matrix complete

        // x^T fragments (tokens 32 ks + 8 g + slot) of this wave's 16 columns,
        // decay-matrix fragments, x for the D term, and w_j
        Frag xf[2], mf[4][2];
        float xv[4][4], w[2][8];
        O::template tr2<0, 32 * PX, 4 * PX>(O::tr_addr(sX, PX, 8 * g, 16 * wave, q), xf[0], xf[1]);
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mf[it][ks] = O::mrow(sM, MP, 16 * it + q, 32 * ks + 8 * g);
#pragma unroll
        for (int it = 0; it < 4; ++it) O::load4(sX, PX, 16 * it + q, 16 * wave + 4 * g, xv[it]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) w[ks][sl] = sW[kTile * kt + 32 * ks + 8 * g + sl];

        // (6) intra-chunk term Y^T += x^T . M^T (zeros above the diagonal)
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc[it] = O::mma(acc[it], xf[ks], mf[it][ks]);

        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NST > 1) {
            fetch_xd((step + NST - 1) % NST, fk, fm, fkt);
            if (fk < nch) advance(fk, fm, fkt);
        }
        if (last_m) {
            // (3) chunk state h += B^T . (w o x)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                Frag bt[NT];
                tr_tiles<O, NT, ES, 4 * PB>(O::tr_addr_pairs(sB, PB, 32 * ks + 8 * g, q), bt);
                const Frag xw = O::scale(xf[ks], w[ks]);
#pragma unroll
                for (int t = 0; t < NT; ++t) st[t] = O::mma(st[t], bt[t], xw);
            }
        }

        // stores: y of M-tile m (written on diagonal steps; 4 instructions every
        // step), then the state after the chunk's last token into its slot
        {
            const bool ystore = (kt == m);
            const int vm = min(kTile, Lc - kTile * m);
            const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(yg + ((t0 + kTile * m) * H + h) * P + p0), 0, ystore ? vm * xrow : 0, kBufFlags);
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                float yv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) yv[r] = acc[it][r] + Dh * xv[it][r];
                O::store_y(ry, (16 * it + q) * xrow + (16 * wave + 4 * g) * ES, yv);
            }
            const bool bad_slot = dst >= a.capacity;
            if (bad_slot && tid == 0) atomicOr(a.error_flag, SSD_DATA_BAD_SLOT);
            dst = __builtin_amdgcn_readfirstlane(bad_slot ? -1 : dst);
            ex2 = ex1;
            ex1 = dst >= 0;
            if (dst >= 0) {
                float *cbase = a.chunk_states + ((int64_t)dst * H + h) * P * N + (int64_t)p0 * N;
                const __amdgpu_buffer_rsrc_t re =
                    __builtin_amdgcn_make_buffer_rsrc((void *)cbase, 0, SH::kCols * N * 4, kBufFlags);
                const int eoff = (16 * wave + q) * N * 4;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, st[t]), re,
                                                           state_n(t) < N ? eoff + 4 * state_n(t) : kOob, 0, 0);
            }
        }
        if constexpr (NST == 1) lds_barrier();   // the single stage is refilled next step
        advance(k, m, kt);
    }

    float *fd = a.final_states + ((int64_t)(s * H + h) * P + pw + q) * N;
#pragma unroll
    for (int t = 0; t < NT; ++t)
        if (state_n(t) < N) *reinterpret_cast<f32x4 *>(fd + state_n(t)) = st[t];
}
#endif

template <typename T, int NW, int N>
hipError_t launch_scan_instance(const ScanArgs &a, hipStream_t stream) {
    using SH = ScanShape<T, NW, N>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&ssd_scan_kernel<T, NW, N>),
        hipFuncAttributeMaxDynamicSharedMemorySize, SH::kLdsBytes);
    if (attr != hipSuccess) return attr;
    const int64_t blocks = (int64_t)a.S * a.H * a.nptiles;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((ssd_scan_kernel<T, NW, N>), dim3((unsigned)blocks), dim3(SH::kThreads),
                       SH::kLdsBytes, stream, a, a.chunk_state_dst);
    return hipGetLastError();
}

template <typename T, int N>
hipError_t launch_scan_waves(const ScanArgs &a, int waves, hipStream_t stream) {
    switch (waves) {
    case 1: return launch_scan_instance<T, 1, N>(a, stream);
    case 2: return launch_scan_instance<T, 2, N>(a, stream);
    case 4: return launch_scan_instance<T, 4, N>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
