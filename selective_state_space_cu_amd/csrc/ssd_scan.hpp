// Fused tile-walk kernel of the Mamba2 SSD varlen scan for gfx950.
//
// One workgroup owns one (sequence, head, headdim tile of 16*NW columns) and
// walks that sequence's tokens in tiles, in order; each of its NW waves owns
// 16 headdim columns and carries their (16 x N) float32 state in registers
// from tile to tile, so states never round-trip through HBM (only exported
// checkpoints and final states are written).
//
// Tiles hold min(chunk_size, 64) tokens. A chunk longer than 64 tokens is
// walked as consecutive 64-token tiles with the state passed between them:
// the chunked form is an exact re-association of the recurrence, so this is
// the same linear map as the quadratic form over the whole chunk, with less
// work. chunk_size still fixes the chunk grid and which states are exported
// (the state after the last token of each chunk).
//
// Per tile (the chunked decomposition of the SSD layer; the numbers follow the
// kernel list of the problem statement):
//   (2) delta_j = softplus(dt_j + dt_bias), cumulative log-decay s_j =
//       sum_{k<=j} delta_k*A (inclusive, tile-local, log2 units) and per-token
//       factors, computed one tile ahead of their use;
//   (5) CB^T = B . C^T per 16x16 sub-tile on the matrix cores, masked by the
//       segment-sum decay: M[i][j] = CB[i][j] * 2^(s_i - s_j) * delta_j for
//       j <= i, plus D on the diagonal (the skip term D x rides with (6));
//   (6) Y^T = h_in . C^T scaled per token by 2^(s_i)   (inter-chunk term)
//           + x^T . M^T                                (intra-chunk and D terms);
//   (3,4) h_out = 2^(s_last) h_in + B^T . (w o x),  w_j = delta_j 2^(s_last - s_j).
// The decay that reaches the entering state at token i is 2^(s_i) with s_i the
// INCLUSIVE cumsum at i, and the total decay is read at the tile's last valid
// token (s is constant past it, since delta is 0 there) -- never past the
// sequence end (the init-state decay rule of the varlen bug-fix page).
//
// Decay matrix: on a diagonal 16x16 sub-tile the factor is 2^(s_i - s_j)
// itself, masked for j > i. Below the diagonal (row block I > column block J)
// it is split at the ends of blocks J and I-1:
//   2^(s_i - s_j) delta_j = V_i * P(I, J) * B_j,  V_i = 2^(s_i - s_end(I-1)),
//   P(I, J) = 2^(s_end(I-1) - s_end(J)),  B_j = delta_j 2^(s_end(J) - s_j),
// each factor at most 1 for a decaying state (A <= 0), so nothing overflows,
// and each element costs two multiplies instead of an exp2. Sub-tiles above
// the diagonal get P = 0.
//
// Memory pipeline: the B, C and x tiles of step i + NST - 1 (and the dt of the
// tile after it) are fetched with direct-to-LDS buffer loads during step i
// (NST stage buffers). Every step issues the same number of vector memory
// instructions (out-of-range buffer lanes are zero-filled on load and dropped
// on store), so an exact s_waitcnt vmcnt(n) waits for one stage only. The
// direct loads are issued through inline assembly: the compiler does not see
// them, so none of its LDS reads waits for them (it would otherwise wait for
// all of them before every transposed read); the stage hand-off is ordered by
// those exact waits and the barrier after them. The step loop is unrolled over
// the NST stages, so LDS addresses are per-lane bases plus immediates.
//
// LDS layouts (conflict-free for the reads that dominate):
//   C tile: rows padded by 16 bytes, so the 16 rows of a row-fragment read
//           start on 16 distinct 16-byte bank groups;
//   B tile: rows padded by 32 bytes plus 128 bytes after every 8 rows, so the
//           eight rows {0..3, 8..11} (or {4..7, 12..15}) that one transposed
//           read touches start on eight distinct 32-byte bank groups;
//   x tile: rows padded by 16 bytes.
//
// Operand layouts on the matrix cores (v_mfma_f32_16x16x32_bf16; the f32 path
// issues eight v_mfma_f32_16x16x4f32 per 32-deep step with the same
// fragments): lane l = 16*g + q supplies row/column q and the 8 "k slots" of
// group g. Any assignment of k indices to (g, slot) is valid as long as both
// operands use the same one, which lets
//   - token-major tiles in LDS feed operands that contract over tokens through
//     the gfx950 LDS transpose read (ds_read_b64_tr_b16), and
//   - the carried state, held in the accumulator layout of B^T.(w o x), feed
//     the inter-chunk product directly from registers: its k slots take n in
//     the order the accumulator tiles hold it (4 rows of one tile, then 4 of
//     the next), and C is read in that order; C . B^T reads B the same way and
//     shares the C fragments.
// Row blocks are visited in the order ib[d] = (wave + d) mod 4, so for the
// decay-matrix column block J = wave the offset d from the diagonal is a
// compile-time index: d = 0 is the diagonal (mask and D term) and every wave
// runs the same code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssd_internal.h"

namespace ssd {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kTile = 64;       // tokens per tile
constexpr int kLdsLimit = 160 * 1024;
constexpr int kBufFlags = 0x00020000;  // raw buffer resource word 3 on gfx9-family parts
constexpr int kOob = 0x40000000;       // buffer offset beyond every tile's range (zero fill / dropped)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

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

// Direct-to-LDS buffer loads: lane l's 16 (or 4) bytes land at LDS byte
// address lds + 16 l (or + 4 l). Issued through inline assembly (see the
// memory pipeline note above), with a raw buffer resource made of wave-uniform
// words: base address, num_records bytes (loads past it read zero), stride 0.
__device__ __forceinline__ u32x4 dma_rsrc(const void *base, int num_records) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu)),
                 (uint32_t)__builtin_amdgcn_readfirstlane(num_records), (uint32_t)kBufFlags};
}
// gfx9 parts need one wait state between a scalar write of M0 and an LDS-DMA
// load that reads it, and five between a VALU write of an SGPR (the
// readfirstlane of a resource word) and a vector memory instruction reading it.
// The compiler pads its own code for both but cannot see inside this asm, so
// the asm carries them itself: s_mov m0 + s_nop 4 is six wait states before the
// load, whatever precedes the asm. Without them a load may take the previous
// M0 (landing on the previous block's LDS address) or a stale resource word.
// Each load carries the stage buffer it fills as an assembly comment
// ("ssd-stage k"), and each explicit wait the stage it releases ("ssd-wait k"),
// so that a check of the compiled code can count, on every path, the vector
// memory instructions between a stage's last load and the wait that releases
// it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int STAGE>
__device__ __forceinline__ void dma16(const u32x4 &r, uint32_t lds, int voff) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds ; ssd-stage %3"
                 :: "v"(voff), "s"(r), "s"(lds), "i"(STAGE) : "memory", "m0");
}
template <int STAGE>
__device__ __forceinline__ void dma4(const u32x4 &r, uint32_t lds, int voff) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds ; ssd-stage %3"
                 :: "v"(voff), "s"(r), "s"(lds), "i"(STAGE) : "memory", "m0");
}
// Wait until at most VM vector memory instructions of this wave are
// outstanding; on gfx9 parts loads and stores count in one counter and retire
// in issue order, so this releases every load issued VM or more instructions
// before the wait.
// EXCL of the VM instructions are checkpoint-export stores, issued on the
// steps the kernel counted as exporting (tagged "ssd-export").
template <int VM, int STAGE, int EXCL = 0>
__device__ __forceinline__ void wait_vm_stage() {
    static_assert(VM >= 0 && VM <= 63, "vmcnt out of range");
    asm volatile("s_waitcnt vmcnt(%0) ; ssd-wait %1 excl %2" :: "i"(VM), "i"(STAGE), "i"(EXCL) : "memory");
}
// A 16-byte store of a checkpoint (exported chunk state): `off` is the byte
// offset into the buffer resource r (offsets past its size are dropped).
// gfx940-family parts (gfx950 included) need two wait states between a store
// of more than 8 bytes and a VALU write of its data registers (the compiler
// pads its own stores, not this asm, and reuses the registers at once), hence
// the s_nop 1.
__device__ __forceinline__ void export_store16(const u32x4 &v, const u32x4 &r, int off) {
    asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen ; ssd-export\n\ts_nop 1" :: "v"(v), "v"(off), "s"(r) : "memory");
}
// The same with the non-temporal + sc1 cache policy (written once, not re-read).
__device__ __forceinline__ void export_store16_nt(const u32x4 &v, const u32x4 &r, int off) {
    asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen nt sc1 ; ssd-export\n\ts_nop 1" :: "v"(v), "v"(off), "s"(r) : "memory");
}
// Placeholder stores through a zero-sized buffer resource (dropped by the
// hardware). Written in assembly so that the compiler can neither merge nor
// eliminate them: they exist only to keep the number of vector memory
// instructions per pipeline step fixed.
__device__ __forceinline__ void null_store8(const u32x4 &r) {
    asm volatile("buffer_store_dwordx2 %0, off, %1, 0" :: "v"(u32x2{0, 0}), "s"(r) : "memory");
}
__device__ __forceinline__ void null_store16(const u32x4 &r) {   // (s_nop: see export_store16)
    asm volatile("buffer_store_dwordx4 %0, off, %1, 0\n\ts_nop 1" :: "v"(u32x4{0, 0, 0, 0}), "s"(r) : "memory");
}
#pragma clang diagnostic pop

// ---------------------------------------------------------------------------
// Element traits: fragment type, LDS fragment reads, matrix op.
// ---------------------------------------------------------------------------
template <typename T> struct Ops;

// bfloat16 (stored as uint16_t)
template <> struct Ops<uint16_t> {
    struct Frag { u32x4 w; };
    static constexpr int kPad = 16;      // decay matrix row padding (elements): 160-byte rows
    static constexpr int kHiOff = 32;    // bytes from the low to the high half of a permuted row fragment

    __device__ static f32x4 mma(f32x4 acc, const Frag &a, const Frag &b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.w),
                                                       __builtin_bit_cast(bf16x8, b.w), acc, 0, 0, 0);
    }
    // Row fragment in the permuted 32-deep k order of lane group g: slots 0..3
    // <- row[k0 + 4g ..], slots 4..7 <- row[k0 + 16 + 4g ..]; p points at
    // row[k0 + 4g]. The two halves are read as separate 8-byte loads (volatile,
    // so they are not merged into one two-address read: on this layout two
    // single reads cost a quarter of the merged one's bank cycles).
    __device__ static Frag rowk_perm(const unsigned char *p) {
        typedef const volatile __attribute__((address_space(3))) u32x2 lds_u32x2;
        const uint32_t la = lds_addr(p);
        const u32x2 lo = *(lds_u32x2 *)(uintptr_t)la;
        const u32x2 hi = *(lds_u32x2 *)(uintptr_t)(la + kHiOff);
        return Frag{u32x4{lo.x, lo.y, hi.x, hi.y}};
    }
    // Transposed fragment of a token-major tile (gfx950 ds_read_b64_tr_b16):
    // slots s <- tile[kb + s][column of the lane]. Within each 16-lane group,
    // lane q supplies the 4 elements at row kb + q/4, columns 4(q%4)..+3 of the
    // group's 16 columns, and receives column q of rows kb..kb+3; a fragment is
    // two such reads (rows kb.. and kb+4.., `four_rows` bytes apart). The
    // lane's first address is row kb + tr_row(q), column col0 + tr_col(q).
    __device__ static int tr_row(int q) { return q >> 2; }
    __device__ static int tr_col(int q) { return 4 * (q & 3); }
    __device__ static Frag tr(const unsigned char *p, int four_rows) {
        const uint32_t la = lds_addr(p);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)la);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)(la + four_rows));
        const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
        return Frag{u32x4{a.x, a.y, b.x, b.y}};
    }
    // decay-matrix row fragment: slots s <- m[k + s] (p points at it)
    __device__ static Frag mrow(const unsigned char *p) { return Frag{*reinterpret_cast<const u32x4 *>(p)}; }
    __device__ static void mstore4(unsigned char *p, const float (&v)[4]) {
        *reinterpret_cast<u32x2 *>(p) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    }
    __device__ static Frag from_f32(const f32x4 &lo, const f32x4 &hi) {
        return Frag{u32x4{pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]), pack_bf16(hi[0], hi[1]),
                          pack_bf16(hi[2], hi[3])}};
    }
    __device__ static Frag scale(const Frag &f, const float (&w)[8]) {
        Frag r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.w[i] = pack_bf16(bf16_lo(f.w[i]) * w[2 * i], bf16_hi(f.w[i]) * w[2 * i + 1]);
        return r;
    }
    // 4 output values (consecutive headdim columns) -> y
    __device__ static void store_y(__amdgpu_buffer_rsrc_t r, int off, const f32x4 &v) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, r, off, 0, 0);
    }
};

// float32
template <> struct Ops<float> {
    struct Frag { float v[8]; };
    static constexpr int kPad = 8;       // 288-byte rows
    static constexpr int kHiOff = 64;

    __device__ static f32x4 mma(f32x4 acc, const Frag &a, const Frag &b) {
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
        return acc;
    }
    __device__ static Frag rowk_perm(const unsigned char *p) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(p + kHiOff);
        return Frag{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
    }
    // column reads: slot s <- tile[kb + s][col0 + q] (rows four_rows / 4 bytes apart)
    __device__ static int tr_row(int) { return 0; }
    __device__ static int tr_col(int q) { return q; }
    __device__ static Frag tr(const unsigned char *p, int four_rows) {
        Frag f;
#pragma unroll
        for (int s = 0; s < 8; ++s) f.v[s] = *reinterpret_cast<const float *>(p + s * (four_rows / 4));
        return f;
    }
    __device__ static Frag mrow(const unsigned char *p) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 16);
        return Frag{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
    }
    __device__ static void mstore4(unsigned char *p, const float (&v)[4]) {
        *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    }
    __device__ static Frag from_f32(const f32x4 &lo, const f32x4 &hi) {
        return Frag{{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}};
    }
    __device__ static Frag scale(const Frag &f, const float (&w)[8]) {
        Frag r;
#pragma unroll
        for (int s = 0; s < 8; ++s) r.v[s] = f.v[s] * w[s];
        return r;
    }
    __device__ static void store_y(__amdgpu_buffer_rsrc_t r, int off, const f32x4 &v) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
    }
};

// Tile shapes and the LDS plan of one (dtype, waves, dstate) instance.
template <typename T, int NW, int N>
struct ScanShape {
    static constexpr int kThreads = 64 * NW;
    static constexpr int kCols = 16 * NW;            // headdim columns per workgroup
    static constexpr int kES = sizeof(T);
    static constexpr int kNE = N < 32 ? 32 : N;      // state width in LDS / registers (zero-padded)
    static constexpr int kRG = N * kES;              // bytes per B/C row in global memory
    static constexpr int kRB = kNE * kES;            // data bytes per B/C tile row in LDS
    static constexpr int kRX = kCols * kES;          // data bytes per x tile row
    static constexpr int kPC = kRB + 16;             // C row pitch
    static constexpr int kPB = kRB + 32;             // B row pitch within a group of 8 rows
    static constexpr int kGB = 8 * kPB + 128;        // B bytes per group of 8 rows
    static constexpr int kPX = kRX + 16;             // x row pitch
    static constexpr int kTileC = kTile * kPC;       // all multiples of 1 KB
    static constexpr int kTileB = 8 * kGB;
    static constexpr int kTileX = kTile * kPX;
    static constexpr int kIC = (kTileC / 1024 + NW - 1) / NW;   // 1 KB direct loads per wave (C)
    static constexpr int kIB = (kTileB / 1024 + NW - 1) / NW;   // (B)
    static constexpr int kIX = (kTileX / 1024 + NW - 1) / NW;   // (x)
    static constexpr int kLoads = kIC + kIB + kIX + 1;          // + one dt load: vector memory loads per wave per step
    static constexpr int kNT = kNE / 16;                        // 16-row state tiles (even)
    static constexpr int kYStores = 4;                          // y stores per wave per step
    static constexpr int kNK = kNE / 32;                        // 32-deep steps over dstate
    static constexpr int kMP = kTile + Ops<T>::kPad;            // decay matrix pitch (elements)
    static constexpr int kMPB = kMP * kES;
    // scan tables of one tile: S, E, Dl, W, V, Bf (64 floats each) and P (16)
    static constexpr int kTab = 6 * 64 + 16;
    static constexpr int kStage = kTileC + kTileB + kTileX + 256;
    static constexpr int kSink = 2048 + 1024;
    static constexpr int bytes(int n) { return n * (kStage + kTab * 4) + kTile * kMPB + kSink; }
    static constexpr bool fit(int n) { return bytes(n) <= kLdsLimit; }
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
    static_assert(fit(1), "tile does not fit in LDS");
    // byte offset of row r in a B tile
    __device__ static int brow(int r) { return (r >> 3) * kGB + (r & 7) * kPB; }
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
__device__ __forceinline__ float readlane(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// softplus(u) = max(u, 0) + ln(1 + e^-|u|), on the hardware exp2/log2
__device__ __forceinline__ float softplus_hw(float u) {
    const float z = fast_exp2(-fabsf(u) * kLog2e);
    return fmaxf(u, 0.0f) + __builtin_amdgcn_logf(1.0f + z) * 0.6931471805599453f;
}

// Scan tables of one tile from delta (lane j = token j; delta = 0 past the tile
// end): S = s_j, E = 2^(s_j), Dl = delta_j, W = delta_j 2^(s_last - s_j),
// V = 2^(s_j - s_end(block(j) - 1)), Bf = delta_j 2^(s_end(block(j)) - s_j)
// (64 floats each, block = 16 tokens, s_end(-1) = 0), and
// P[4 J + d] = 2^(s_end(J + d - 1) - s_end(J)) for 1 <= d and J + d < 4, 0 for
// J + d >= 4 (16 floats). Every wave computes the scan (a short latency
// chain); wave w stores the entries of its share of the lanes and the other
// lanes store into `sink` (2 KB of scratch LDS).
template <int NW>
__device__ __forceinline__ void tile_tables(float *tab, float *sink, float d, float a2, int lane, int wave) {
    const float v = wave_scan(d * a2);
    const float e0 = readlane(v, 15), e1 = readlane(v, 31), e2 = readlane(v, 47), e3 = readlane(v, 63);
    const int blk = lane >> 4;
    const float s_prev = blk == 0 ? 0.0f : (blk == 1 ? e0 : (blk == 2 ? e1 : e2));
    const float s_end = blk == 0 ? e0 : (blk == 1 ? e1 : (blk == 2 ? e2 : e3));
    const bool owner = ((lane * NW) >> 6) == wave;
    float *p = owner ? tab + lane : sink + lane;
    p[0] = v;
    p[64] = fast_exp2(v);
    p[128] = d;
    p[192] = d * fast_exp2(e3 - v);
    p[256] = fast_exp2(v - s_prev);
    p[320] = d * fast_exp2(s_end - v);
    // P, by lanes 4 J + d < 16 of wave 0
    const int J = (lane >> 2) & 3, dd = lane & 3, I = J + dd;
    const float ea = I == 1 ? e0 : (I == 2 ? e1 : e2), eb = J == 0 ? e0 : (J == 1 ? e1 : e2);
    const float pv = dd == 0 ? 1.0f : (I >= 4 ? 0.0f : fast_exp2(ea - eb));
    float *pp = (wave == 0 && lane < 16) ? tab + 384 + lane : sink + 384 + lane;
    *pp = pv;
}

// Workgroup -> (sequence rank, head, headdim tile). Workgroups are handed to
// the 8 XCDs round-robin (block b runs on XCD b mod 8), each with its own L2,
// and within an XCD in block order (sequence ranks ascend, so the longest
// sequences start first on every XCD). Mappings (ScanArgs::xcd_mode):
//   kXcdPairs: all workgroups of one (sequence, group) pair -- which read the
//     same B and C tiles -- land on one XCD, pairs p = x, x + 8, ... on XCD x.
//     Every XCD gets the same work when G is a multiple of 8 (XCD x takes
//     groups x, x + 8, ... of every sequence) or when all sequences have the
//     same length.
//   kXcdSplit: every XCD takes 1/8 of each sequence's workgroups, a contiguous
//     run of heads (so a group's B and C tiles are read by as few XCDs as
//     this balance allows): the same work on every XCD for any length mix.
//   kXcdPairsIfEqual (kXcdPairsIfEqualElseNone): kXcdPairs when all sequence
//     lengths are equal, else kXcdSplit (kXcdNone); decided here from
//     cu_seqlens, every wave gets the same answer.
//   kXcdNone: block order (sequence rank, head, tile); consecutive heads of a
//     sequence go to different XCDs.
__device__ __forceinline__ bool all_lengths_equal(const ScanArgs &a) {
    const int lane = threadIdx.x & 63;
    const int l0 = a.cu_seqlens[1] - a.cu_seqlens[0];
    bool eq = true;
    for (int i = lane; i < a.S; i += 64) eq = eq && (a.cu_seqlens[i + 1] - a.cu_seqlens[i]) == l0;
    return __builtin_amdgcn_ballot_w64(!eq) == 0;
}
__device__ __forceinline__ void decode_block(const ScanArgs &a, int b, int &rank, int &h, int &pt) {
    int mode = a.xcd_mode;
    if (mode == kXcdPairsIfEqual || mode == kXcdPairsIfEqualElseNone)
        mode = all_lengths_equal(a) ? kXcdPairs : (mode == kXcdPairsIfEqual ? kXcdSplit : kXcdNone);
    const int x = b & 7, i = b >> 3;
    if (mode == kXcdPairs) {
        const int hpg = a.H / a.G;
        const int wpp = hpg * a.nptiles;   // workgroups per pair
        const int pair = x + 8 * (i / wpp), loc = i - (i / wpp) * wpp;
        rank = pair / a.G;
        h = (pair - rank * a.G) * hpg + loc / a.nptiles;
        pt = loc - (loc / a.nptiles) * a.nptiles;
    } else if (mode == kXcdSplit) {
        const int per_x = a.H * a.nptiles / 8;   // workgroups of one sequence per XCD
        rank = i / per_x;
        const int loc = x * per_x + (i - rank * per_x);
        h = loc / a.nptiles;
        pt = loc - h * a.nptiles;
    } else {
        const int per_seq = a.H * a.nptiles;
        rank = b / per_seq;
        const int rem = b - rank * per_seq;
        h = rem / a.nptiles;
        pt = rem - h * a.nptiles;
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
    constexpr int NST = SH::kNST, RG = SH::kRG, RX = SH::kRX, PC = SH::kPC, PB = SH::kPB, PX = SH::kPX;
    constexpr int ES = SH::kES, NT = SH::kNT, NK = SH::kNK, MPB = SH::kMPB, TAB = SH::kTab;
    constexpr int JS = 4 / NW;   // decay-matrix column blocks per wave
    static_assert(NW == 1 || NW == 2 || NW == 4, "1, 2 or 4 waves per workgroup");

    // Separate LDS objects, so the compiler knows that decay-matrix and table
    // stores never alias tile reads and may reorder them freely.
    __shared__ __align__(16) unsigned char sC[NST * SH::kTileC];
    __shared__ __align__(16) unsigned char sB[NST * SH::kTileB];
    __shared__ __align__(16) unsigned char sX[NST * SH::kTileX];
    __shared__ __align__(16) float sDt[NST * 64];
    __shared__ __align__(16) unsigned char sM[kTile * MPB];
    __shared__ __align__(16) float tabs[NST * TAB + 512];   // + 2 KB of discarded table stores
    __shared__ __align__(16) float sink_dma[256];          // discarded direct loads (1 KB)
    float *const sink = tabs + NST * TAB;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (kept in an SGPR)
    const int q = lane & 15, g = lane >> 4;

    if (__builtin_nontemporal_load(a.error_flag) & SSD_DATA_BAD_CU_SEQLENS) return;
    int rank, h, pt;
    decode_block(a, blockIdx.x, rank, h, pt);
    const int s = a.seq_order[rank];
    if (s < 0 || s >= a.S) return;
    const int grp = h / (a.H / a.G);
    const int H = a.H, P = a.P, G = a.G, cs = a.cs;
    int64_t tb = a.cu_seqlens[s], te = a.cu_seqlens[s + 1];
    tb = tb < 0 ? 0 : (tb > a.T ? a.T : tb);
    te = te < tb ? tb : (te > a.T ? a.T : te);
    const int L = (int)(te - tb);
    const int TT = cs < kTile ? cs : kTile;   // tokens per tile
    const int nt = (L + TT - 1) / TT;         // tiles of this sequence
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
    const int xrow = H * P * ES;    // bytes between tokens of x / y
    const int browg = G * N * ES;   // bytes between tokens of B / C

    auto tile_len = [&](int t) { return min(TT, L - t * TT); };
    // the state after tile t is exported when the tile ends a chunk: its slot, else -1
    auto slot_of = [&](int t) -> int {
        if (a.chunk_states == nullptr || t >= nt) return -1;
        if (((t + 1) * TT) % cs != 0 && t != nt - 1) return -1;
        const int gc = c0 + (t * TT) / cs;
        return (gc >= 0 && gc < a.max_chunks) ? (dstmap ? dstmap[gc] : gc) : -1;
    };

    // Carried state, in the accumulator layout of B^T . (w o x): st[t][r] = h[p = pw + q][n = 16 t + 4 g + r].
    // The pair st[2c], st[2c+1] is the 32-deep operand of step c of C . h^T in the
    // permuted k order (slots 0..3: n = 32 c + 4 g + r, slots 4..7: n = 32 c + 16 + 4 g + r),
    // so C is read in that order, and C . B^T shares those C fragments.
    // Rows n >= N (dstate < 32 only) stay zero.
    f32x4 st[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) st[u] = f32x4{0, 0, 0, 0};
    auto state_n = [&](int u) { return 16 * u + 4 * g; };
    if (a.init != nullptr && (a.has_init == nullptr || a.has_init[s] != 0)) {
        const float *src = a.init + ((int64_t)(s * H + h) * P + pw + q) * N;
#pragma unroll
        for (int u = 0; u < NT; ++u)
            if (state_n(u) < N) st[u] = *reinterpret_cast<const f32x4 *>(src + state_n(u));
    }

    // scan tables of tile 0, from global dt
    if (nt > 0) {
        float d = 0.0f;
        if (lane < tile_len(0)) d = softplus_hw(a.dt[(tb + lane) * H + h] + bias);
        tile_tables<NW>(tabs, sink, d, a2, lane, wave);
    }
    __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);   // nothing outstanding before the tile pipeline starts

    // Per-lane parts of the direct-to-LDS loads (loop invariant). Lane l of load
    // block j fills LDS bytes [1024 j + 16 l, +16) of a tile; bytes of row
    // padding (and past dstate in global memory) get an out-of-range offset.
    struct GlobalOffsets { int c[SH::kIC], b[SH::kIB], x[SH::kIX]; int d; } go;
#pragma unroll
    for (int i = 0; i < SH::kIC; ++i) {
        const int j = wave + NW * i, o = 1024 * j + 16 * lane, r = o / PC, pos = o % PC;
        go.c[i] = (j < SH::kTileC / 1024 && pos < RG) ? r * browg + pos : kOob;
    }
#pragma unroll
    for (int i = 0; i < SH::kIB; ++i) {
        const int j = wave + NW * i, o = 1024 * j + 16 * lane;
        const int gr = o / SH::kGB, rm = o % SH::kGB, rin = rm / PB, pos = rm % PB;
        go.b[i] = (j < SH::kTileB / 1024 && rin < 8 && pos < RG) ? (8 * gr + rin) * browg + pos : kOob;
    }
#pragma unroll
    for (int i = 0; i < SH::kIX; ++i) {
        const int j = wave + NW * i, o = 1024 * j + 16 * lane, r = o / PX, pos = o % PX;
        go.x[i] = (j < SH::kTileX / 1024 && pos < RX) ? r * xrow + pos : kOob;
    }
    go.d = wave == 0 ? lane * H * 4 : kOob;
    // LDS byte addresses (integers: no generic pointers in the address arithmetic)
    const uint32_t lds_sink = lds_addr(sink_dma), lds_c = lds_addr(sC), lds_b = lds_addr(sB),
                   lds_x = lds_addr(sX), lds_dt = lds_addr(sDt);
    auto lds_u = [&](uint32_t a) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)a); };

    // Fetch the tiles of tile u into stage buffer SLOT (out-of-range,
    // zero-filling loads when u >= nt): part 0 loads C and B, part 1 x and the
    // dt of tile u + 1; always kLoads instructions per wave in all. The parts
    // are issued at different points of a step, so that the waves of a
    // workgroup do not all queue their loads at the same moment.
    auto fetch = [&](auto part, auto slot_c, int u) {
        constexpr int PART = decltype(part)::value, SLOT = decltype(slot_c)::value;
        const bool live = u < nt;
        const int Lt = live ? tile_len(u) : 0;
        const int64_t t0 = tb + (int64_t)u * TT;
        if constexpr (PART == 0) {
            const u32x4 rC = dma_rsrc(Cg + (t0 * G + grp) * N, Lt * browg);
            const u32x4 rB = dma_rsrc(Bg + (t0 * G + grp) * N, Lt * browg);
#pragma unroll
            for (int i = 0; i < SH::kIC; ++i) {
                const int j = wave + NW * i;   // 1 KB block of the tile
                dma16<SLOT>(rC, lds_u(j < SH::kTileC / 1024 ? lds_c + SLOT * SH::kTileC + 1024 * j : lds_sink), go.c[i]);
            }
#pragma unroll
            for (int i = 0; i < SH::kIB; ++i) {
                const int j = wave + NW * i;
                dma16<SLOT>(rB, lds_u(j < SH::kTileB / 1024 ? lds_b + SLOT * SH::kTileB + 1024 * j : lds_sink), go.b[i]);
            }
        } else {
            const u32x4 rX = dma_rsrc(xg + (t0 * H + h) * P + p0, Lt * xrow);
            const bool dnext = live && u + 1 < nt;
            const u32x4 rD = dma_rsrc(a.dt + (dnext ? t0 + TT : 0) * H + h, dnext ? tile_len(u + 1) * H * 4 : 0);
#pragma unroll
            for (int i = 0; i < SH::kIX; ++i) {
                const int j = wave + NW * i;
                dma16<SLOT>(rX, lds_u(j < SH::kTileX / 1024 ? lds_x + SLOT * SH::kTileX + 1024 * j : lds_sink), go.x[i]);
            }
            dma4<SLOT>(rD, lds_u(wave == 0 ? lds_dt + SLOT * 256 : lds_sink), go.d);
        }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // y stores of a step that writes no y (keeps the per-step count fixed):
    // kYStores stores of y's width through a zero-sized resource
    const u32x4 r_none = dma_rsrc(yg, 0);
    auto dummy_y_stores = [&]() {
#pragma unroll
        for (int i = 0; i < SH::kYStores; ++i) {
            if constexpr (sizeof(T) == 2) null_store8(r_none);
            else null_store16(r_none);
        }
    };
    // wait for stage SLOT; `exports` = checkpoint exports among the last NST-1 steps
    auto wait_stage = [&](auto slot_c, int exports) {
        constexpr int SLOT = decltype(slot_c)::value;
        if constexpr (NST == 3) {
            if (exports == 0) wait_vm_stage<SH::vm_wait(3, 0), SLOT>();
            else if (exports == 1) wait_vm_stage<SH::vm_wait(3, 1), SLOT, SH::kNT>();
            else wait_vm_stage<SH::vm_wait(3, 2), SLOT, 2 * SH::kNT>();
        } else if constexpr (NST == 2) {
            if (exports == 0) wait_vm_stage<SH::vm_wait(2, 0), SLOT>();
            else wait_vm_stage<SH::vm_wait(2, 1), SLOT, SH::kNT>();
        }
    };

    // prologue: stages of tiles 0 .. NST-2
    if constexpr (NST > 1) {
        fetch(P0{}, std::integral_constant<int, 0>{}, 0);
        fetch(P1{}, std::integral_constant<int, 0>{}, 0);
        dummy_y_stores();
    }
    if constexpr (NST > 2) {
        fetch(P0{}, std::integral_constant<int, 1>{}, 1);
        fetch(P1{}, std::integral_constant<int, 1>{}, 1);
        dummy_y_stores();
    }

    // Row blocks of the Y^T tiles in visiting order: acc[d] covers tile rows
    // 16 ib[d] + q. The decay-matrix sub-tile of column block jb = wave + NW jj at
    // offset dd below the diagonal has row block (jb + dd) mod 4 = ib[(NW jj + dd) mod 4].
    int ib[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) ib[d] = (wave + d) & 3;
    // diagonal sub-tiles: the causal mask as an exponent bias, and D on the diagonal
    float cm[4], dadd[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        cm[r] = 4 * g + r <= q ? 0.0f : -INFINITY;
        dadd[r] = 4 * g + r == q ? Dh : 0.0f;
    }

    f32x4 acc[4];   // Y^T tiles: acc[d][r] = y[token 16 ib[d] + q][p = pw + 4 g + r]
    int ex1 = 0, ex2 = 0;   // did the previous / second previous step export a state
    int dst = slot_of(0);   // checkpoint slot of the state after the current tile, or -1
    int t = 0;              // current tile

    // One step: tile t in stage SLOT (= t mod NST).
    auto step = [&](auto slot_c) {
        constexpr int SLOT = decltype(slot_c)::value;
        constexpr int NEXT = (SLOT + 1) % NST, FETCH = (SLOT + NST - 1) % NST;
        const unsigned char *tC = sC + SLOT * SH::kTileC;
        const unsigned char *tB = sB + SLOT * SH::kTileB;
        const unsigned char *tX = sX + SLOT * SH::kTileX;
        const float *tab = tabs + SLOT * TAB;
        const float *tS = tab, *tE = tab + 64, *tD = tab + 128, *tW = tab + 192, *tV = tab + 256, *tBf = tab + 320,
                    *tP = tab + 384;
        const int Lt = tile_len(t);
        const int64_t t0 = tb + (int64_t)t * TT;

        if constexpr (NST == 1) {
            fetch(P0{}, slot_c, t);
            fetch(P1{}, slot_c, t);
            __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);
        } else {
            wait_stage(slot_c, NST == 3 ? ex1 + ex2 : ex1);
        }
        lds_barrier();   // (A) stage SLOT and this tile's scan tables are visible

        // ---- phase A: the LDS operands of the step, then the matrix work
        const float sL = tS[63];   // total log-decay of the tile (s is constant past its end)
        // C fragments of the row blocks (32-deep k steps over n in the permuted
        // order of the state), shared by the inter-chunk product and C . B^T
        Frag cfm[4][NK];
        float ei[4], vi[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int il = 16 * ib[d] + q;
            const unsigned char *pc = tC + il * PC + 4 * g * ES;
#pragma unroll
            for (int c = 0; c < NK; ++c) cfm[d][c] = O::rowk_perm(pc + 32 * c * ES);
            ei[d] = tE[il];
            vi[d] = tV[il];
        }
        // B fragments and column factors of this wave's column blocks
        Frag bf[JS][NK];
        float si0[JS], sj[JS][4], dj[JS][4], bj[JS][4], pf[JS][4];
#pragma unroll
        for (int jj = 0; jj < JS; ++jj) {
            const int jb = wave + NW * jj;
            const unsigned char *pb = tB + SH::brow(16 * jb + q) + 4 * g * ES;
#pragma unroll
            for (int c = 0; c < NK; ++c) bf[jj][c] = O::rowk_perm(pb + 32 * c * ES);
            si0[jj] = tS[16 * jb + q];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int jc = 16 * jb + 4 * g + r;
                sj[jj][r] = tS[jc];
                dj[jj][r] = tD[jc];
                bj[jj][r] = tBf[jc];
                pf[jj][r] = tP[4 * jb + r];
            }
        }
        // x^T fragments (tokens 32 ks + 8 g + slot) of this wave's 16 columns, shared by
        // the state update and the intra term, and B^T fragments (tile u: state rows n = 16 u ..)
        Frag xf[2], bt[2][NT];
        float w[2][8];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            xf[ks] = O::tr(tX + (32 * ks + 8 * g + O::tr_row(q)) * PX + (16 * wave + O::tr_col(q)) * ES, 4 * PX);
            const unsigned char *pb = tB + SH::brow(32 * ks + 8 * g) + O::tr_row(q) * PB + O::tr_col(q) * ES;
#pragma unroll
            for (int u = 0; u < NT; ++u) bt[ks][u] = O::tr(pb + 16 * u * ES, 4 * PB);
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) w[ks][sl] = tW[32 * ks + 8 * g + sl];
        }

        // B and C of tile t + NST - 1, into the stage the previous step used
        // (issued after this phase's LDS reads)
        if constexpr (NST > 1) fetch(P0{}, std::integral_constant<int, FETCH>{}, t + NST - 1);

        // (6) inter-chunk term Y^T = h_in . C^T, then scale column i by 2^(s_i)
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[d] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < NK; ++c) {
            const Frag hf = O::from_f32(st[2 * c], st[2 * c + 1]);
#pragma unroll
            for (int d = 0; d < 4; ++d) acc[d] = O::mma(acc[d], hf, cfm[d][c]);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[d] *= ei[d];

        // (3, 4) state: h = 2^(s_last) h + B^T . (w o x)
        {
            const float e = fast_exp2(sL);
#pragma unroll
            for (int u = 0; u < NT; ++u) st[u] *= e;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const Frag xw = O::scale(xf[ks], w[ks]);
#pragma unroll
                for (int u = 0; u < NT; ++u) st[u] = O::mma(st[u], bt[ks][u], xw);
            }
        }

        // (5) decay-matrix sub-tiles (row block ib[dr], column block jb) -> LDS
#pragma unroll
        for (int jj = 0; jj < JS; ++jj) {
            const int jb = wave + NW * jj;
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                const int dr = (NW * jj + dd) & 3;   // visiting index of row block (jb + dd) mod 4
                f32x4 cb = {0, 0, 0, 0};
#pragma unroll
                for (int c = 0; c < NK; ++c) cb = O::mma(cb, bf[jj][c], cfm[dr][c]);
                float v[4];
                if (dd == 0) {   // diagonal: exact factor, masked, plus D
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = fmaf(cb[r], fast_exp2(cm[r] + (si0[jj] - sj[jj][r])) * dj[jj][r], dadd[r]);
                } else {         // below the diagonal (P = 0 for blocks above it)
                    const float rowf = vi[dr] * pf[jj][dd];
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = cb[r] * (rowf * bj[jj][r]);
                }
                O::mstore4(sM + (16 * ib[dr] + q) * MPB + (16 * jb + 4 * g) * ES, v);
            }
        }

        // scan tables of the next tile, from the dt that rode with this stage
        {
            const bool nxt = t + 1 < nt;
            const int Ln = nxt ? tile_len(t + 1) : 0;
            const float dn = softplus_hw(sDt[SLOT * 64 + lane] + bias + (lane < Ln ? 0.0f : -INFINITY));
            tile_tables<NW>(nxt ? tabs + NEXT * TAB : sink, sink, dn, a2, lane, wave);
        }
        lds_barrier();   // (B) decay matrix and next tables complete

        // ---- phase B: (6) intra-chunk and D terms Y^T += x^T . M^T
        Frag mf[4][2];
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mf[d][ks] = O::mrow(sM + (16 * ib[d] + q) * MPB + (32 * ks + 8 * g) * ES);
        if constexpr (NST > 1)   // x and dt of tile t + NST - 1
            fetch(P1{}, std::integral_constant<int, FETCH>{}, t + NST - 1);
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc[d] = O::mma(acc[d], xf[ks], mf[d][ks]);

        // stores: y of the tile (4 instructions), then the state after the tile
        // into its checkpoint slot if the tile ends a chunk
        {
            const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(yg + (t0 * H + h) * P + p0), 0, Lt * xrow, kBufFlags);
#pragma unroll
            for (int d = 0; d < 4; ++d) O::store_y(ry, (16 * ib[d] + q) * xrow + (16 * wave + 4 * g) * ES, acc[d]);
            const bool bad_slot = dst >= a.capacity;
            if (bad_slot && tid == 0) atomicOr(a.error_flag, SSD_DATA_BAD_SLOT);
            const int dsl = __builtin_amdgcn_readfirstlane(bad_slot ? -1 : dst);
            ex2 = ex1;
            ex1 = dsl >= 0;
            if (dsl >= 0) {
                float *cbase = a.chunk_states + ((int64_t)dsl * H + h) * P * N + (int64_t)p0 * N;
                const u32x4 re = dma_rsrc(cbase, SH::kCols * N * 4);
                const int eoff = (16 * wave + q) * N * 4;
#pragma unroll
                for (int u = 0; u < NT; ++u)
                    export_store16(__builtin_bit_cast(u32x4, st[u]), re, state_n(u) < N ? eoff + 4 * state_n(u) : kOob);
            }
        }
        if constexpr (NST == 1) lds_barrier();   // the single stage is refilled next step
        ++t;
        // slot of the next tile's state (loaded now, so that no scalar load is in
        // flight while the next step reads LDS)
        dst = slot_of(t);
    };

    while (t < nt) {
        step(std::integral_constant<int, 0>{});
        if constexpr (NST > 1) {
            if (t >= nt) break;
            step(std::integral_constant<int, 1>{});
        }
        if constexpr (NST > 2) {
            if (t >= nt) break;
            step(std::integral_constant<int, 2>{});
        }
    }

    float *fd = a.final_states + ((int64_t)(s * H + h) * P + pw + q) * N;
#pragma unroll
    for (int u = 0; u < NT; ++u)
        if (state_n(u) < N) *reinterpret_cast<f32x4 *>(fd + state_n(u)) = st[u];
}
#endif

template <typename T, int NW, int N>
hipError_t launch_scan_instance(const ScanArgs &a, hipStream_t stream) {
    using SH = ScanShape<T, NW, N>;
    const int64_t blocks = (int64_t)a.S * a.H * a.nptiles;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((ssd_scan_kernel<T, NW, N>), dim3((unsigned)blocks), dim3(SH::kThreads), 0, stream, a,
                       a.chunk_state_dst);
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
