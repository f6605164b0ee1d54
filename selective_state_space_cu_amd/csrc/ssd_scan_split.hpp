// Split-state variant of the fused tile-walk scan, for bf16 inputs with
// dstate 128 (the Mamba2 layer shape): two waves per SIMD instead of one.
//
// One workgroup owns one (sequence, head, 64 headdim columns), like the
// four-wave kernel in ssd_scan.hpp, but runs eight waves: wave w owns the 16
// columns of block pb = w mod 4 and HALF nh = w / 4, meaning
//   - state rows n in [nh N/2, (nh + 1) N/2) of those columns (float32, in
//     registers, carried from tile to tile), and
//   - output tokens 32 nh .. 32 nh + 31 of every tile (y rows, decay-matrix rows).
// Waves w and w + 4 run on the same SIMD, so each SIMD interleaves two
// instruction streams and hides the latency a single wave would stall on.
//
// The inter-chunk term of a wave's 32 tokens needs the whole entering state of
// its 16 columns, so the two halves are swapped once per tile: after the state
// update each wave converts its half to the bf16 operand fragments of the next
// tile's inter-chunk product and stores them into the C-tile blocks of the
// stage it has just consumed (those bytes are dead until the same reader
// refills them with its own direct loads, after reading the fragments), and
// its partner reads them after the next tile's first barrier.
//
// Per tile, wave (pb, nh), row blocks I = 2 nh + d (d = 0, 1), column block J = pb:
//   Y^T[p, i]   = h_in[p, :] . C[i, :]^T                (all n: own + partner halves)
//   CB[i, j]    = C[i, :] . B[j, :]^T -> decay matrix M[i, j] (sub-tiles (I, J))
//   h_out[p, n] = 2^(s_last) h_in[p, n] + sum_j B[j, n] w_j x[j, p]  (own n half)
//   Y^T[p, i]  += sum_j x[j, p] M[i, j]                 (after the second barrier)
// with the scan tables (s, 2^s, delta, w) of the next tile computed by waves 0-3
// (and, after the second barrier, each wave's decay factors of the next tile).
// The tile pipeline (NST stages, exact vmcnt waits) is that of the four-wave
// kernel for B, C and dt (direct-to-LDS loads two tiles ahead). x, the stream
// that comes from HBM, runs deeper through registers: each wave loads its 1 KB
// of x for tile t + 5 at the end of step t and writes it into the stage three
// steps later, once that stage has been consumed (4 VGPRs per step of depth
// instead of another 41 KB stage).
//
// LDS tiles are unpadded (a C or B tile is 16 KB, an x tile 8 KB, so each of
// the eight waves fills whole 1 KB blocks of every tile) and conflict-free by
// an XOR swizzle of 16-byte chunks: chunk k of row r is stored at chunk
// k ^ swz(r). The direct loads apply it on the global side (each lane picks
// the global chunk that belongs at its LDS position); the readers apply it
// per lane. B and C rows (256 bytes) use swz(r) = r mod 16, x rows (128 bytes)
// swz(r) = (b2, b1, b3) of r (bit 0 first).
//
// State layout: lane (g, q) holds h[p][n] for p = pw + q and the 16 n values
// nb + 16 g .. nb + 16 g + 15 (register u, element r: n = nb + 16 g + 4 (u ^ (g & 1)) + r;
// the u ^ (g & 1) order makes the transposed B reads conflict-free). So the
// 32-deep k step c of every product over n takes, in lane group g, the 8
// consecutive n = nb + 16 g + 8 c .. + 7: one 16-byte read per C or B row
// fragment, and the state needs no data movement to become an operand.
//
// Stores leave the workgroup as whole 128-byte lines: each wave puts its y
// values into an LDS tile of the workgroup's 64 tokens x 64 columns, which is
// written out row by row after the next barrier (one step later); a
// checkpoint is transposed through the just-consumed B tile, so that each
// store covers 4 state rows x 256 contiguous bytes.
#pragma once

#include "ssd_scan.hpp"

namespace ssd {

// Direct-to-LDS loads with the LDS address as an SGPR base plus a compile-time
// offset (m0 = base + OFF), so that per-stage addresses need no extra registers;
// one wait state between the M0 write and the load (the gfx9 M0 / LDS-DMA hazard).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// A wave-uniform resource quad as SGPRs (the asm operands below need them;
// readfirstlane is free for a value the compiler already keeps in SGPRs).
__device__ __forceinline__ u32x4 sgpr4(const u32x4 &r) {
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)r.x), (uint32_t)__builtin_amdgcn_readfirstlane((int)r.y),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)r.z), (uint32_t)__builtin_amdgcn_readfirstlane((int)r.w)};
}
// (The "ssd-stage k" comment names the stage the load fills; see dma16.)
template <int OFF, int STAGE>
__device__ __forceinline__ void dma16_at(const u32x4 &r0, uint32_t lds_base, int voff) {
    const u32x4 r = sgpr4(r0);
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds ; ssd-stage %4"
                 :: "v"(voff), "s"(r), "s"(lds_base), "i"(OFF), "i"(STAGE) : "memory", "m0", "scc");
}
template <int OFF, int STAGE>
__device__ __forceinline__ void dma4_at(const u32x4 &r0, uint32_t lds_base, int voff) {
    const u32x4 r = sgpr4(r0);
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds ; ssd-stage %4"
                 :: "v"(voff), "s"(r), "s"(lds_base), "i"(OFF), "i"(STAGE) : "memory", "m0", "scc");
}
// A 16-byte buffer load into registers that the compiler does not track (like
// the direct-to-LDS loads): the caller waits for it with an explicit vmcnt and
// then passes the value through reg_fence, so that no use moves above the wait.
// The compiler takes the destination as written at once, so on EVERY path from
// the load the value must stay live until a wait covers it: a path on which it
// is dead (an early return, a skipped store) lets the compiler give those
// registers to other values, which the late load then overwrites. The CPU
// tests check the compiled code for this (first touch of the registers on
// every path is their LDS store, or a vmcnt(0) wait comes first).
template <int OFF, int STAGE>
__device__ __forceinline__ void load16_untracked(u32x4 &dst, const u32x4 &r0, int voff) {
    const u32x4 r = sgpr4(r0);
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen offset:%3 ; ssd-stage %4"
                 : "=v"(dst) : "v"(voff), "s"(r), "i"(OFF), "i"(STAGE) : "memory");
}
__device__ __forceinline__ void reg_fence(u32x4 &v) { asm volatile("" : "+v"(v)); }
#pragma clang diagnostic pop

// Compile-time loop: f(integral_constant<int, i>) for i = 0 .. N-1.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Row fragment: 8 consecutive bf16 (one 16-byte read); transposed fragment:
// two ds_read_b64_tr_b16 from per-lane addresses.
__device__ __forceinline__ Ops<uint16_t>::Frag rf16(uint32_t addr) {
    return Ops<uint16_t>::Frag{*(const __attribute__((address_space(3))) u32x4 *)(uintptr_t)addr};
}
__device__ __forceinline__ Ops<uint16_t>::Frag tr2(uint32_t lo_addr, uint32_t hi_addr) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)lo_addr);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)hi_addr);
    const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
    return Ops<uint16_t>::Frag{u32x4{a.x, a.y, b.x, b.y}};
}
// Orders LDS accesses across the lanes of one wave at the compiler level
// (the hardware executes a wave's LDS instructions in order): values read
// before it are not reused for reads after it.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}
// Cache policy of the y and checkpoint stores (written once, not re-read
// here): non-temporal with the sc1 scope bit, which timed 1-1.5 % faster on the
// prefix-cache workload than non-temporal alone (plain, sc1 alone and sc0 + nt
// were no faster).
constexpr int kStoreNT = 2 | 16;
// Wave-uniform 64-bit value (kept in an SGPR pair).
__device__ __forceinline__ uint64_t uni64(uint64_t v) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
}
// Raw buffer resource: base address, num_records bytes (accesses past it
// read zero / are dropped), stride 0.
__device__ __forceinline__ u32x4 buf_rsrc(uint64_t b, int num_records) {
    return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, (uint32_t)num_records, (uint32_t)kBufFlags};
}

template <int N>
struct SplitShape {
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kCols = 64;                 // headdim columns per workgroup
    static constexpr int kES = 2;                    // bf16
    static constexpr int kRB = N * kES;              // bytes per B/C row (256)
    static constexpr int kRX = kCols * kES;          // bytes per x / y tile row (128)
    static constexpr int kTileC = kTile * kRB;       // 16 KB
    static constexpr int kTileB = kTile * kRB;
    static constexpr int kTileX = kTile * kRX;       // 8 KB
    static constexpr int kIC = kTileC / 1024 / kWaves;   // 1 KB direct loads per wave (C)
    static constexpr int kIB = kTileB / 1024 / kWaves;   // (B)
    static constexpr int kIX = kTileX / 1024 / kWaves;   // (x)
    static constexpr int kLoads = kIC + kIB + kIX + 1;   // + one dt load
    static constexpr int kNKH = N / 64;              // 32-deep steps over one state half
    static constexpr int kNTH = N / 32;              // state registers (f32x4) per lane
    static constexpr int kMPB = (kTile + 16) * kES;  // decay matrix row pitch (160 bytes)
    static constexpr int kTab = 4 * 64;              // S, E, Dl, W
    static constexpr int kStage = kTileC + kTileB + kTileX + 256;
    static constexpr int kStageE = 1024;             // checkpoint staging per wave (4 rows x 256 bytes)
    // stages, decay matrix, y tile, x . w tile, checkpoint staging
    static constexpr int bytes(int n) { return n * (kStage + kTab * 4) + kTile * kMPB + 2 * kTileX + kWaves * kStageE; }
    static constexpr bool fit(int n) { return bytes(n) <= kLdsLimit; }
    // vector memory instructions issued after the last load of the stage
    // waited for: that step's register load of x, then one y store and the
    // next step's loads, and kNTH stores per step that exported a checkpoint
    static constexpr int vm_wait(int exports) { return 2 + kLoads + exports * kNTH; }
    static constexpr int kNST = 3;
    static_assert(fit(kNST), "three stages must fit in LDS");
    static_assert(vm_wait(4) <= 63, "vmcnt range");
    // the partner's state fragments use C blocks w + 8 c of a consumed stage
    static_assert(8 * kNKH <= kTileC / 1024, "state exchange needs 8 C blocks per fragment");
    // a checkpoint is staged in 2 KB per wave of a consumed B tile
    static_assert(N == 128, "the swizzles and layouts are laid out for 256-byte B/C rows");
    __device__ static int swz128(int r) { return ((r >> 2) & 1) | (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2); }
};

// Workgroup -> (sequence rank, first head, headdim tile) when each workgroup
// walks a.items consecutive heads of one (sequence, group) pair (the pair
// mapping of decode_block, with a.items heads per workgroup).
__device__ __forceinline__ void decode_block_multi(const ScanArgs &a, int b, int &rank, int &h0, int &pt) {
    const int hpg = a.H / a.G, K = a.items;
    const int wpp = hpg / K * a.nptiles;   // workgroups per pair
    const int x = b & 7, i = b >> 3;
    const int pair = x + 8 * (i / wpp), loc = i - (i / wpp) * wpp;
    rank = pair / a.G;
    h0 = (pair - rank * a.G) * hpg + (loc / a.nptiles) * K;
    pt = loc - (loc / a.nptiles) * a.nptiles;
}

// MULTI: the workgroup walks the tiles of a.items consecutive heads as one
// stream (same sequence and group, so the same B and C tiles): the pipeline
// runs on from one head into the next, so a head's start-up (initial state,
// first stages, tables) overlaps the previous head's last tiles.
template <int N, bool MULTI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ssd_scan_split_kernel(ScanArgs a, const int32_t *__restrict__ dstmap)
#if !defined(__HIP_DEVICE_COMPILE__)
{   // the host pass only needs the signature (for the launch stub)
}
#else
{
    using O = Ops<uint16_t>;
    using Frag = O::Frag;
    using SH = SplitShape<N>;
    constexpr int NST = SH::kNST, RB = SH::kRB, RX = SH::kRX;
    constexpr int NTH = SH::kNTH, NKH = SH::kNKH, MPB = SH::kMPB, TAB = SH::kTab;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

    __shared__ __align__(16) unsigned char sC[NST * SH::kTileC];
    __shared__ __align__(16) unsigned char sB[NST * SH::kTileB];
    __shared__ __align__(16) unsigned char sX[NST * SH::kTileX];
    __shared__ __align__(16) float sDt[NST * 64];
    __shared__ __align__(16) unsigned char sM[kTile * MPB];
    __shared__ __align__(16) unsigned char sY[SH::kTileX];   // y of the previous tile
    __shared__ __align__(16) float tabs[NST * TAB];
    __shared__ __align__(16) unsigned char sXW[SH::kTileX];   // x . w of the current tile (x tile layout)
    __shared__ __align__(16) unsigned char sE[SH::kWaves * SH::kStageE];   // checkpoint staging

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (kept in an SGPR)
    const int pb = wave & 3, nh = wave >> 2;                      // column block, half
    const int q = lane & 15, g = lane >> 4;
    const bool godd = (g & 1) != 0;

    if (__builtin_nontemporal_load(a.error_flag) & SSD_DATA_BAD_CU_SEQLENS) return;
    int rank, h, pt;   // (with MULTI, h is the workgroup's first head)
    if constexpr (MULTI) decode_block_multi(a, blockIdx.x, rank, h, pt);
    else decode_block(a, blockIdx.x, rank, h, pt);
    const int K = MULTI ? a.items : 1;   // heads walked by this workgroup
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
    // chunk_size and the tile are powers of two: a chunk is 2^lg_tpc tiles
    const int lg_tpc = __builtin_ctz((unsigned)cs) - __builtin_ctz((unsigned)TT);
    const int c0 = a.seq_chunk_start[s];
    const int p0 = pt * SH::kCols;       // first headdim column of the workgroup
    const int pw = p0 + 16 * pb;         // first headdim column of this wave
    const int nb = nh * (N / 2);         // first state row of this wave's half
    const int r0 = 32 * nh;              // first token row of this wave's half
    // (with MULTI: bias and a2 are those of the head whose tables are computed
    // next; lane k of cb_l, ca_l, cd_l holds head h + k's)
    float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    float a2 = a.A[h] * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.0f;
    float cb_l = 0.0f, ca_l = 0.0f, cd_l = 0.0f;
    if constexpr (MULTI) {
        if (lane < K) {
            cb_l = a.dt_bias ? a.dt_bias[h + lane] : 0.0f;
            ca_l = a.A[h + lane] * kLog2e;
            cd_l = a.D ? a.D[h + lane] : 0.0f;
        }
    }
    const int xrow = H * P * 2;     // bytes between tokens of x / y
    const int browg = G * N * 2;    // bytes between tokens of B / C
    const int clampTT = TT;
    auto clamp_len = [&](int rem) { return rem < 0 ? 0 : (rem > clampTT ? clampTT : rem); };

    // The state after tile t is exported when the tile ends a chunk (or is
    // the sequence's last): ex_tile is the next such tile, ex_chunk its chunk.
    const int tpc = 1 << lg_tpc;
    int ex_tile = a.chunk_states != nullptr ? min(tpc, nt) - 1 : nt;
    int ex_chunk = c0;
    // Checkpoint slots of 64 chunks at a time, lane k holding chunk ex_win + k
    // (-1: none), so that an export reads its slot with v_readlane instead of
    // a scalar load whose latency the next barrier would wait for.
    int ex_win = c0;
    auto load_slots = [&](int c) {
        const int gc = c + lane;
        return (gc >= 0 && gc < a.max_chunks) ? (dstmap ? dstmap[gc] : gc) : -1;
    };
    int slots = a.chunk_states != nullptr ? load_slots(ex_win) : -1;
    // n offset (elements) of register u's 4 values within the lane's 16
    auto n_of = [&](int u) { return 16 * g + 4 * (u ^ (g & 1)); };

    // This wave's half of the carried state (see the layout note above).
    f32x4 st[NTH];
#pragma unroll
    for (int u = 0; u < NTH; ++u) st[u] = f32x4{0, 0, 0, 0};
    const bool has_init = a.init != nullptr && (a.has_init == nullptr || a.has_init[s] != 0);
    if (has_init) {
        const float *src = a.init + ((int64_t)(s * H + h) * P + pw + q) * N + nb;
#pragma unroll
        for (int u = 0; u < NTH; ++u) st[u] = *reinterpret_cast<const f32x4 *>(src + n_of(u));
    }
    // MULTI: the initial and final states of head h + k, through buffer
    // resources spanning this sequence's H P N floats (offsets out of that
    // range read zero / are dropped); stn holds the next head's initial state.
    f32x4 stn[NTH];
    const int seq_bytes = H * P * N * 4;
    const uint64_t init_seq = uni64((uint64_t)(uintptr_t)a.init + (uint64_t)s * (uint64_t)seq_bytes);
    const uint64_t fin_seq = uni64((uint64_t)(uintptr_t)a.final_states + (uint64_t)s * (uint64_t)seq_bytes);
    auto state_off = [&](int k, int u) { return (((h + k) * P + pw + q) * N + nb + n_of(u)) * 4; };
    auto load_init = [&](f32x4 (&dst)[NTH], int k) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(uintptr_t)init_seq, 0, has_init && k < K ? seq_bytes : 0, kBufFlags);
#pragma unroll
        for (int u = 0; u < NTH; ++u)
            dst[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, state_off(k, u), 0, 0));
    };
    auto store_final = [&](int k) {   // (NTH stores, counted like a checkpoint export)
        const u32x4 r = buf_rsrc(fin_seq, k < K ? seq_bytes : 0);
#pragma unroll
        for (int u = 0; u < NTH; ++u) export_store16(__builtin_bit_cast(u32x4, st[u]), r, state_off(k, u));
    };
    if constexpr (MULTI) load_init(stn, 1);

    // Scan tables of a tile from delta (lane j = token j; delta = 0 past the
    // tile end), one table per wave of waves 0-3: S = s_j (inclusive cumulative
    // log2-decay), E = 2^(s_j), Dl = delta_j, W = delta_j 2^(s_last - s_j).
    // (wave-uniform float selectors instead of branches)
    const float k_s = wave == 0 ? 1.0f : 0.0f, k_e = wave == 1 ? 1.0f : 0.0f, k_d = wave == 2 ? 1.0f : 0.0f,
                k_w = wave == 3 ? 1.0f : 0.0f;
    auto tables = [&](float *tab, float d) {
        const float v = wave_scan(d * a2);
        const float e3 = readlane(v, 63);
        const float ex = fast_exp2(k_e * v + (1.0f - k_e) * (e3 - v));   // 2^(s_j), or 2^(s_last - s_j)
        tab[64 * wave + lane] = k_s * v + (k_e + k_w * d) * ex + k_d * d;
    };
    if (nt > 0 && wave < 4) {
        float d = 0.0f;
        if (lane < clamp_len(L)) d = softplus_hw(a.dt[(tb + lane) * H + h] + bias);
        tables(tabs, d);
    }

    // Exchange of state halves: the fragments this wave gives its partner
    // (wave ^ 4) go to C blocks (wave ^ 4) + 8 c of a consumed stage, which the
    // partner reads before it refills them. Fragment c, lane group g: the 8
    // values n = nb + 16 g + 8 c .. + 7 (registers 2c, 2c+1 in g-dependent order).
    Frag hown[NKH];
    auto make_own = [&]() {
#pragma unroll
        for (int c = 0; c < NKH; ++c) {
            const uint32_t a0 = pack_bf16(st[2 * c][0], st[2 * c][1]), a1 = pack_bf16(st[2 * c][2], st[2 * c][3]);
            const uint32_t b0 = pack_bf16(st[2 * c + 1][0], st[2 * c + 1][1]),
                           b1 = pack_bf16(st[2 * c + 1][2], st[2 * c + 1][3]);
            hown[c].w = godd ? u32x4{b0, b1, a0, a1} : u32x4{a0, a1, b0, b1};
        }
    };
    const uint32_t x_put = lds_addr(sC) + 1024 * (wave ^ 4) + 16 * lane;
    const uint32_t x_get = lds_addr(sC) + 1024 * wave + 16 * lane;
    auto put_own = [&](auto slot_c) {
        constexpr int SLOT = decltype(slot_c)::value;
#pragma unroll
        for (int c = 0; c < NKH; ++c) *(lds_u32x4 *)(uintptr_t)(x_put + SLOT * SH::kTileC + 8192 * c) = hown[c].w;
    };
    make_own();
    put_own(std::integral_constant<int, NST - 1>{});   // read by step 0 (from stage NST - 1)
    __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);        // nothing outstanding before the tile pipeline starts

    // Per-lane parts of the direct-to-LDS loads (loop invariant): lane l of
    // load block j fills LDS bytes [1024 j + 16 l, +16) of a tile, i.e. chunk
    // l mod 16 (l mod 8 for x) of row 4 j + l / 16 (8 j + l / 8), with the
    // global chunk that the swizzle puts there.
    int go_c[SH::kIC], go_b[SH::kIB], go_x[SH::kIX];
#pragma unroll
    for (int i = 0; i < SH::kIC; ++i) {
        const int r = 4 * (wave + 8 * i) + (lane >> 4);
        go_c[i] = r * browg + 16 * ((lane & 15) ^ (r & 15));
    }
#pragma unroll
    for (int i = 0; i < SH::kIB; ++i) {
        const int r = 4 * (wave + 8 * i) + (lane >> 4);
        go_b[i] = r * browg + 16 * ((lane & 15) ^ (r & 15));
    }
#pragma unroll
    for (int i = 0; i < SH::kIX; ++i) {
        const int r = 8 * (wave + 8 * i) + (lane >> 3);
        go_x[i] = r * xrow + 16 * ((lane & 7) ^ SH::swz128(r));
    }
    const int go_d = lane * H * 4;   // every wave loads the same dt (identical bytes)
    // LDS byte addresses of this wave's first 1 KB block in each tile region
    // (wave-uniform); block i of stage SLOT is at + SLOT * tile + 8 KB i
    auto rfl = [&](uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); };
    const uint32_t lds_c = rfl(lds_addr(sC) + 1024 * wave), lds_b = rfl(lds_addr(sB) + 1024 * wave),
                   lds_x = rfl(lds_addr(sX) + 1024 * wave), lds_dt = rfl(lds_addr(sDt));

    // Running global positions of the tile being fetched (tile f) and of the
    // tile whose y is being stored (tile t - 1).
    // (buffer resources kept as loop-carried SGPR quads: per tile, the base
    // address advances and num_records is set to the tile's bytes)
    u32x4 r_c = buf_rsrc(uni64((uint64_t)(uintptr_t)a.C + (uint64_t)((tb * G + grp) * N) * 2), 0);
    u32x4 r_b = buf_rsrc(uni64((uint64_t)(uintptr_t)a.B + (uint64_t)((tb * G + grp) * N) * 2), 0);
    u32x4 r_x = buf_rsrc(uni64((uint64_t)(uintptr_t)a.x + (uint64_t)((tb * H + h) * P + p0) * 2), 0);
    u32x4 r_d = buf_rsrc(uni64((uint64_t)(uintptr_t)a.dt + (uint64_t)((tb + TT) * H + h) * 4), 0);
    int f_rem = L;                         // tokens from tile f on
    const uint32_t step_bc = (uint32_t)__builtin_amdgcn_readfirstlane(TT * browg),
                   step_x = (uint32_t)__builtin_amdgcn_readfirstlane(TT * xrow),
                   step_d = (uint32_t)__builtin_amdgcn_readfirstlane(TT * H * 4);
    auto advance = [](u32x4 &r, uint32_t inc) {   // base += inc (48-bit address, stride bits stay 0)
        const uint64_t v = (((uint64_t)r.y) << 32 | r.x) + inc;
        r.x = (uint32_t)v;
        r.y = (uint32_t)(v >> 32);
    };
    // MULTI: stream positions (head k, tile) of the fetch cursor; the dt that
    // rides with a stage is that of the stream's next tile (d_rem its tokens)
    int fi = 0, ft = 0, d_rem = 0;
    auto next_pos = [&](int &k, int &tl) {
        if (++tl == nt) { tl = 0; ++k; }
    };
    auto set_fetch = [&]() {
        const int64_t tok = tb + (int64_t)ft * TT;
        r_c = buf_rsrc(uni64((uint64_t)(uintptr_t)a.C + (uint64_t)((tok * G + grp) * N) * 2), 0);
        r_b = buf_rsrc(uni64((uint64_t)(uintptr_t)a.B + (uint64_t)((tok * G + grp) * N) * 2), 0);
        r_x = buf_rsrc(uni64((uint64_t)(uintptr_t)a.x + (uint64_t)((tok * H + h + fi) * P + p0) * 2), 0);
        int di = fi, dtl = ft;
        next_pos(di, dtl);
        r_d = buf_rsrc(uni64((uint64_t)(uintptr_t)a.dt + (uint64_t)((tb + (int64_t)dtl * TT) * H + h + di) * 4), 0);
        f_rem = fi < K ? L - ft * TT : 0;
        d_rem = di < K ? L - dtl * TT : 0;
    };
    if constexpr (MULTI) set_fetch();

    // Fetch tile f into stage buffer SLOT (zero-filling loads past the
    // sequence): part 0 loads C and B, part 1 x and the dt of tile f + 1
    // (then advances f); always kLoads instructions per wave in all.
    auto fetch = [&](auto part, auto slot_c, auto with_x) {
        constexpr int PART = decltype(part)::value, SLOT = decltype(slot_c)::value;
        const int Lt = clamp_len(f_rem);
        if constexpr (PART == 0) {
            r_c.z = r_b.z = (uint32_t)(Lt * browg);
            static_for<SH::kIC>([&](auto i_c) {
                constexpr int I = decltype(i_c)::value;
                dma16_at<SLOT * SH::kTileC + 8192 * I, SLOT>(r_c, lds_c, go_c[I]);
            });
            static_for<SH::kIB>([&](auto i_c) {
                constexpr int I = decltype(i_c)::value;
                dma16_at<SLOT * SH::kTileB + 8192 * I, SLOT>(r_b, lds_b, go_b[I]);
            });
        } else {
            r_x.z = (uint32_t)(Lt * xrow);
            r_d.z = (uint32_t)(clamp_len(MULTI ? d_rem : f_rem - TT) * H * 4);
            if constexpr (decltype(with_x)::value) {
                static_for<SH::kIX>([&](auto i_c) {
                    constexpr int I = decltype(i_c)::value;
                    dma16_at<SLOT * SH::kTileX + 8192 * I, SLOT>(r_x, lds_x, go_x[I]);
                });
            }
            dma4_at<SLOT * 256, SLOT>(r_d, lds_dt, go_d);
            // next tile (past the sequence end the positions are never dereferenced)
            if constexpr (MULTI) {
                next_pos(fi, ft);
                set_fetch();
            } else {
                advance(r_c, step_bc); advance(r_b, step_bc); advance(r_x, step_x); advance(r_d, step_d);
                f_rem -= TT;
            }
        }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using WithX = std::true_type;
    using NoX = std::false_type;
    static_assert(SH::kIX == 1, "one 1 KB block of x per wave per tile");
    // x of tile t + 5 goes into register set t mod 3 at the end of step t and
    // from there into its stage in step t + 3 (tiles 0 and 1 by direct loads)
    u32x4 xr[NST];
    u32x4 r_xg = buf_rsrc(uni64((uint64_t)(uintptr_t)a.x + (uint64_t)(((tb + 2 * TT) * H + h) * P + p0) * 2), 0);
    int xg_rem = L - 2 * TT;   // tokens from the tile whose x is loaded next
    int xi = 0, xt = 0;        // (MULTI) its stream position
    auto set_xg = [&]() {
        r_xg = buf_rsrc(uni64((uint64_t)(uintptr_t)a.x +
                              (uint64_t)(((tb + (int64_t)xt * TT) * H + h + xi) * P + p0) * 2), 0);
        xg_rem = xi < K ? L - xt * TT : 0;
    };
    if constexpr (MULTI) {
        if (nt > 0) { next_pos(xi, xt); next_pos(xi, xt); }
        else xi = K;
        set_xg();
    }
    auto xload = [&](auto set_c) {
        constexpr int SET = decltype(set_c)::value;
        r_xg.z = (uint32_t)(clamp_len(xg_rem) * xrow);
        load16_untracked<0, SET>(xr[SET], r_xg, go_x[0]);   // waited for by the step of slot SET
        if constexpr (MULTI) {
            next_pos(xi, xt);
            set_xg();
        } else {
            advance(r_xg, step_x);
            xg_rem -= TT;
        }
    };
    // wait for stage SLOT (and the x registers of its set); `exports` =
    // checkpoint exports among the last two steps
    auto wait_stage = [&](auto slot_c, int exports) {
        constexpr int SLOT = decltype(slot_c)::value;
        if (exports == 0) wait_vm_stage<SH::vm_wait(0), SLOT>();
        else if (exports == 1) wait_vm_stage<SH::vm_wait(1), SLOT, NTH>();
        else if (!MULTI || exports == 2) wait_vm_stage<SH::vm_wait(2), SLOT, 2 * NTH>();
        else if (exports == 3) wait_vm_stage<SH::vm_wait(3), SLOT, 3 * NTH>();
        else wait_vm_stage<SH::vm_wait(4), SLOT, 4 * NTH>();
    };

    // y of the previous tile: LDS tile (row rho = token, 128 bytes, chunk k at
    // k ^ ((rho >> 1) & 7)) -> y, one row per 8 lanes
    // tile t - 1 (starts one tile before the sequence, never dereferenced)
    uint64_t y_prev = uni64((uint64_t)(uintptr_t)a.y + (uint64_t)((tb * H + h) * P + p0) * 2 - step_x);
    int y_len = 0;    // its tokens (0: nothing to store)
    int y_rem = L;    // tokens from tile t on
    const int yrow = 8 * wave + (lane >> 3);
    const uint32_t y_get = lds_addr(sY) + yrow * RX + 16 * ((lane & 7) ^ ((yrow >> 1) & 7));
    const uint32_t y_put = lds_addr(sY) + (r0 + q) * RX + 16 * ((2 * pb + (g >> 1)) ^ (((r0 + q) >> 1) & 7)) + 8 * (g & 1);
    auto store_prev_y = [&](const u32x4 &v) {
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)y_prev, 0, y_len * xrow, kBufFlags);
        __builtin_amdgcn_raw_buffer_store_b128(v, ry, yrow * xrow + 16 * (lane & 7), 0, kStoreNT);
    };

    // prologue: stages of tiles 0 .. NST-2 (and the y store slot of step -1)
    xload(std::integral_constant<int, 0>{});   // x of tile 2
    fetch(P0{}, std::integral_constant<int, 0>{}, WithX{});
    fetch(P1{}, std::integral_constant<int, 0>{}, WithX{});
    xload(std::integral_constant<int, 1>{});   // x of tile 3
    null_store16(buf_rsrc(y_prev, 0));   // zero-sized: keeps the per-step count of vector memory ops
    fetch(P0{}, std::integral_constant<int, 1>{}, WithX{});
    fetch(P1{}, std::integral_constant<int, 1>{}, WithX{});
    xload(std::integral_constant<int, 2>{});   // x of tile 4

    // Diagonal structure of this wave's decay-matrix sub-tiles (rows
    // i = r0 + 16 d + q, columns j = 16 pb + 4 g + r): exponent bias 0 for
    // j <= i, -inf above the diagonal; D where j == i.
    float mbias[2][4], dadd[2][4];
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = r0 + 16 * d + q, j = 16 * pb + 4 * g + r;
            mbias[d][r] = j <= i ? 0.0f : -INFINITY;
            dadd[d][r] = j == i ? Dh : 0.0f;
        }

    // Decay factors of this wave's sub-tiles (f = 2^(s_i - s_j) delta_j: at most
    // delta_j for j <= i, 2^(-inf) = 0 above the diagonal) and the inter-chunk
    // row scales 2^(s_i) of a tile, computed from its tables after the barrier
    // before the one that starts its step, off that step's critical path
    float fdec[2][4], eic[2];
    auto decay_of = [&](const float *tab) {
        const float *tS = tab, *tE = tab + 64, *tD = tab + 128;
        float sj[4], dj[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sj[r] = tS[16 * pb + 4 * g + r];
            dj[r] = tD[16 * pb + 4 * g + r];
        }
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            eic[d] = tE[r0 + 16 * d + q];
            const float si = tS[r0 + 16 * d + q];
#pragma unroll
            for (int r = 0; r < 4; ++r) fdec[d][r] = fast_exp2(si - sj[r] + mbias[d][r]) * dj[r];
        }
    };
    auto pin_decay = [&]() {   // keeps the computation where it is written
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            asm volatile("" : "+v"(eic[d]));
#pragma unroll
            for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(fdec[d][r]));
        }
    };

    // Per-lane LDS addresses of the swizzled fragment reads (stage 0; stages,
    // row blocks and k-steps over tokens are immediate offsets).
    //   C rows r0 + q and B rows 16 pb + q: 16 bytes at n = nb' + 16 g + 8 c
    //   (nb' = this wave's or the partner's half)
    const int nbp = N / 2 - nb;
    uint32_t ac_o[NKH], ac_p[NKH], ab_o[NKH], ab_p[NKH];
#pragma unroll
    for (int c = 0; c < NKH; ++c) {
        ac_o[c] = lds_addr(sC) + (r0 + q) * RB + 16 * ((nb / 8 + 2 * g + c) ^ q);
        ac_p[c] = lds_addr(sC) + (r0 + q) * RB + 16 * ((nbp / 8 + 2 * g + c) ^ q);
        ab_o[c] = lds_addr(sB) + (16 * pb + q) * RB + 16 * ((nb / 8 + 2 * g + c) ^ q);
        ab_p[c] = lds_addr(sB) + (16 * pb + q) * RB + 16 * ((nbp / 8 + 2 * g + c) ^ q);
    }
    //   transposed reads of B^T for register u: lane q of each 16-lane group
    //   supplies row kb + q / 4 (+ 4), the 4 values at n = nb + 16 (q mod 4) + 4 (u ^ (q mod 2));
    //   of x^T: row kb + q / 4 (+ 4), columns 16 pb + 4 (q mod 4); kb = 32 ks + 8 g
    uint32_t abt[NTH][2], axf[2];
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
        const int r = 8 * g + (q >> 2) + 4 * hi;
#pragma unroll
        for (int u = 0; u < NTH; ++u) {
            const int byte = 2 * nb + 32 * (q & 3) + 8 * (u ^ (q & 1));
            abt[u][hi] = lds_addr(sB) + r * RB + 16 * ((byte >> 4) ^ (r & 15)) + (byte & 15);
        }
        axf[hi] = lds_addr(sX) + r * RX + 16 * ((2 * pb + ((q >> 1) & 1)) ^ SH::swz128(r)) + 8 * (q & 1);
    }
    // Held as whole per-lane addresses: left visible, the compiler factors them
    // into shared row and swizzle parts and re-adds those in every step.
#pragma unroll
    for (int c = 0; c < NKH; ++c) {
        asm volatile("" : "+v"(ac_o[c]), "+v"(ac_p[c]), "+v"(ab_o[c]), "+v"(ab_p[c]));
    }
#pragma unroll
    for (int u = 0; u < NTH; ++u) asm volatile("" : "+v"(abt[u][0]), "+v"(abt[u][1]));
    int nexp = 0;           // checkpoint exports among the last two steps
    int ex1 = 0;            // did the previous step export
    // the x . w pass: lane 64 wave + lane scales one 16-byte chunk (8 headdim
    // columns of token row xw_row) of the swizzled x tile, in place of layout
    const int xw_row = (64 * wave + lane) >> 3;
    const uint32_t xw_off = xw_row * RX + 16 * (lane & 7);
    // (whole addresses, so that the stage offsets fit the LDS instructions' immediates)
    uint32_t xw_src = lds_addr(sX) + xw_off, xw_dst = lds_addr(sXW) + xw_off;
    uint32_t axw[2] = {axf[0] - lds_addr(sX) + lds_addr(sXW), axf[1] - lds_addr(sX) + lds_addr(sXW)};
    asm volatile("" : "+v"(xw_src), "+v"(xw_dst), "+v"(axw[0]), "+v"(axw[1]));
    // checkpoint staging: 4 state rows x 256 bytes per round, chunk m of row
    // i at m ^ i; round r holds the lanes' rows q = 4 r .. 4 r + 3, and its
    // store reads row lane / 16, chunk lane mod 16
    const uint32_t e_base = lds_addr(sE) + SH::kStageE * wave;
    const uint32_t e_get = e_base + 256 * (lane >> 4) + 16 * ((lane & 15) ^ (lane >> 4));
    int t = 0;              // current tile (of the stream, with MULTI)
    const int ntot = nt * K;  // tiles of the stream
    int ic = 0, tc = 0;       // head (of the workgroup's K) and tile of tile t
    // checkpoint slots: a.chunk_states + slot * H P N floats + this workgroup's block
    uint64_t ck_base = uni64((uint64_t)(uintptr_t)a.chunk_states + (uint64_t)((h * P + p0) * N) * 4);
    const uint64_t ck_slot = uni64((uint64_t)H * P * N * 4);

    // One step: tile t in stage SLOT (= t mod NST).
    auto step = [&](auto slot_c) {
        constexpr int SLOT = decltype(slot_c)::value;
        constexpr int NEXT = (SLOT + 1) % NST, FETCH = (SLOT + NST - 1) % NST;
        constexpr int OC = SLOT * SH::kTileC, OB = SLOT * SH::kTileB, OX = SLOT * SH::kTileX;
        const float *tab = tabs + SLOT * TAB;
        const float *tS = tab, *tW = tab + 192;

        // checkpoint slot of the state after this tile, or -1
        int dsl = -1;
        if ((MULTI ? tc : t) == ex_tile) {
            if (ex_chunk - ex_win >= 64) {   // next window (once per 64 checkpoints)
                ex_win = ex_chunk;
                slots = load_slots(ex_win);
                // wait here, on this rare path, so that no later use of the
                // window waits for vector memory (the pipeline's loads included)
                __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);
            }
            dsl = __builtin_amdgcn_readlane(slots, ex_chunk - ex_win);
            if (dsl >= a.capacity) {
                if (tid == 0) atomicOr(a.error_flag, SSD_DATA_BAD_SLOT);
                dsl = -1;
            }
            dsl = __builtin_amdgcn_readfirstlane(dsl);
            ++ex_chunk;
            ex_tile = min(ex_tile + tpc, nt - 1);
        }

        wait_stage(slot_c, nexp);
        reg_fence(xr[SLOT]);   // x of tile t + 2, loaded three steps ago
        lds_barrier();   // (A) stage SLOT, this tile's tables, the partner's state half and y of tile t-1 are visible

        // ---- phase A
        const u32x4 yv = *(const lds_u32x4 *)(uintptr_t)y_get;   // y of tile t - 1
        Frag hp[NKH];   // the partner's half of h_in, from the C blocks of stage FETCH
#pragma unroll
        for (int c = 0; c < NKH; ++c) hp[c].w = *(const lds_u32x4 *)(uintptr_t)(x_get + FETCH * SH::kTileC + 8192 * c);
        const float sL = tS[63];   // total log-decay of the tile (s is constant past its end)
        // C fragments of this wave's row blocks (own / partner n half) and B
        // fragments of column block pb, shared by C . h^T and C . B^T
        Frag co[2][NKH], cp[2][NKH], bo[NKH], bq[NKH];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
#pragma unroll
            for (int c = 0; c < NKH; ++c) {
                co[d][c] = rf16(ac_o[c] + OC + 16 * RB * d);
                cp[d][c] = rf16(ac_p[c] + OC + 16 * RB * d);
            }
        }
#pragma unroll
        for (int c = 0; c < NKH; ++c) {
            bo[c] = rf16(ab_o[c] + OB);
            bq[c] = rf16(ab_p[c] + OB);
        }
        // (3) x . w of this tile, once per workgroup, for the state update
        // after the next barrier: w_j = delta_j 2^(s_last - s_j) per token row
        {
            const u32x4 xv = *(const lds_u32x4 *)(uintptr_t)(xw_src + OX);
            const float wr = tW[xw_row];
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = pack_bf16(bf16_lo(xv[i]) * wr, bf16_hi(xv[i]) * wr);
            *(lds_u32x4 *)(uintptr_t)xw_dst = o;
        }

        // (6) inter-chunk term Y^T = h_in . C^T over all n, then scale column i by 2^(s_i)
        // (raised wave priority while the matrix products issue: of the two waves
        // on a SIMD, the one feeding the matrix core goes first)
        __builtin_amdgcn_s_setprio(1);
        f32x4 acc[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            acc[d] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < NKH; ++c) {
                acc[d] = O::mma(acc[d], hown[c], co[d][c]);
                acc[d] = O::mma(acc[d], hp[c], cp[d][c]);
            }
            acc[d] *= eic[d];
        }
        store_prev_y(yv);

        // (5) decay-matrix sub-tiles (row block 2 nh + d, column block pb) -> LDS
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            f32x4 cb = {0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < NKH; ++c) {
                cb = O::mma(cb, bo[c], co[d][c]);
                cb = O::mma(cb, bq[c], cp[d][c]);
            }
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = fmaf(cb[r], fdec[d][r], dadd[d][r]);
            O::mstore4(sM + (r0 + 16 * d + q) * MPB + (16 * pb + 4 * g) * 2, v);
        }
        __builtin_amdgcn_s_setprio(0);

        // B and C of tile t + NST - 1 into stage FETCH, once this wave's reads
        // of its C blocks there (the partner's state half) have completed
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        fetch(P0{}, std::integral_constant<int, FETCH>{}, NoX{});

        // scan tables of the next tile, from the dt that rode with this stage
        if (wave < 4 && t + 1 < (MULTI ? ntot : nt)) {
            const int tn = MULTI ? (tc + 1 < nt ? tc + 1 : 0) : t + 1;   // tile index of tile t + 1
            if constexpr (MULTI) {   // that tile's head
                const int kn = tc + 1 < nt ? ic : ic + 1;
                bias = readlane(cb_l, kn);
                a2 = readlane(ca_l, kn);
            }
            const int Ln = clamp_len(L - tn * TT);
            tables(tabs + NEXT * TAB, softplus_hw(sDt[SLOT * 64 + lane] + bias + (lane < Ln ? 0.0f : -INFINITY)));
        }
        lds_barrier();   // (B) decay matrix, x . w and next tables complete; stage SLOT's C tile consumed

        // ---- phase B
        // (4) this wave's state half: h = 2^(s_last) h + B^T . (w o x)
        Frag xf[2];   // x^T fragments (tokens 32 ks + ..) of this wave's columns, for the intra term
        {
            Frag bt[2][NTH], xw[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                xf[ks] = tr2(axf[0] + OX + 32 * RX * ks, axf[1] + OX + 32 * RX * ks);
                xw[ks] = tr2(axw[0] + 32 * RX * ks, axw[1] + 32 * RX * ks);
#pragma unroll
                for (int u = 0; u < NTH; ++u) bt[ks][u] = tr2(abt[u][0] + OB + 32 * RB * ks, abt[u][1] + OB + 32 * RB * ks);
            }
            decay_of(tabs + NEXT * TAB);   // of the next tile (its tables are visible since the last barrier)
            const float e = fast_exp2(sL);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int u = 0; u < NTH; ++u) st[u] *= e;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int u = 0; u < NTH; ++u) st[u] = O::mma(st[u], bt[ks][u], xw[ks]);
            __builtin_amdgcn_s_setprio(0);
        }
        // this wave's half of h_out for the partner, into stage SLOT's C blocks
        make_own();
        put_own(slot_c);
        // (6) intra-chunk and D terms Y^T += x^T . M^T
        Frag mf[2][2];
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mf[d][ks] = O::mrow(sM + (r0 + 16 * d + q) * MPB + (32 * ks + 8 * g) * 2);
        fetch(P1{}, std::integral_constant<int, FETCH>{}, NoX{});   // dt of tile t + NST
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc[d] = O::mma(acc[d], xf[ks], mf[d][ks]);
        // y of this tile -> LDS (stored by the next step)
#pragma unroll
        for (int d = 0; d < 2; ++d)
            *(lds_u32x2 *)(uintptr_t)(y_put + 16 * RX * d) =
                u32x2{pack_bf16(acc[d][0], acc[d][1]), pack_bf16(acc[d][2], acc[d][3])};
        // x of tile t + 2 into stage FETCH (consumed by the previous step)
        *(lds_u32x4 *)(uintptr_t)(lds_x + FETCH * SH::kTileX + 16 * lane) = xr[SLOT];
        if constexpr (MULTI) {
            y_prev = uni64((uint64_t)(uintptr_t)a.y + (uint64_t)(((tb + (int64_t)tc * TT) * H + h + ic) * P + p0) * 2);
            y_len = clamp_len(L - tc * TT);
        } else {
            y_prev += step_x;
            y_len = clamp_len(y_rem);
            y_rem -= TT;
        }

        // the state half after the tile into its checkpoint slot, if the tile
        // ends a chunk: four rounds of 4 state rows through the wave's staging
        // area, each store 4 rows x 256 bytes
        // (MULTI: the last tile of a head that is not the workgroup's last also
        // stores that head's final state: NTH more stores, counted as an export)
        const bool bnd = MULTI && tc == nt - 1 && ic + 1 < K;
        const int ex = (dsl >= 0 ? 1 : 0) + (bnd ? 1 : 0);
        nexp = ex1 + ex;
        ex1 = ex;
        if (dsl >= 0) {
            const uint64_t cbase = ck_base + (uint64_t)dsl * ck_slot;
            const u32x4 re = buf_rsrc(cbase, SH::kCols * N * 4);
#pragma unroll
            for (int rnd = 0; rnd < 4; ++rnd) {
                if ((q >> 2) == rnd) {
#pragma unroll
                    for (int u = 0; u < NTH; ++u) {
                        const int i = q & 3, m = n_of(u) / 4;
                        *(lds_u32x4 *)(uintptr_t)(e_base + 256 * i + 16 * (m ^ i)) = __builtin_bit_cast(u32x4, st[u]);
                    }
                }
                wave_lds_sync();
                const u32x4 v = *(const lds_u32x4 *)(uintptr_t)e_get;
                export_store16_nt(v, re, ((16 * pb + 4 * rnd + (lane >> 4)) * N + nb) * 4 + 16 * (lane & 15));
                wave_lds_sync();
            }
        }
        if constexpr (MULTI) {
            if (bnd) {
                // head ic is done: its final state out, the next head's initial
                // state in (and to the partner, in place of h_out), its D on the
                // diagonal, its checkpoint columns; the chunk walk restarts
                store_final(ic);
#pragma unroll
                for (int u = 0; u < NTH; ++u) st[u] = stn[u];
                load_init(stn, ic + 2);
                make_own();
                put_own(slot_c);
                const float dn = readlane(cd_l, ic + 1);
#pragma unroll
                for (int d = 0; d < 2; ++d)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dadd[d][r] = (16 * pb + 4 * g + r == r0 + 16 * d + q) ? dn : 0.0f;
                ck_base += (uint64_t)P * N * 4;
                ex_tile = a.chunk_states != nullptr ? min(tpc, nt) - 1 : nt;
                ex_chunk = c0;
                if (a.chunk_states != nullptr && ex_win != c0) {
                    ex_win = c0;
                    slots = load_slots(ex_win);
                    __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);
                }
            }
        }
        pin_decay();
        xload(slot_c);   // x of tile t + 5 (set SLOT is free again)
        ++t;
        if constexpr (MULTI) next_pos(ic, tc);
    };

    lds_barrier();   // tile 0's tables are visible
    decay_of(tabs);
    while (t < ntot) {
        step(std::integral_constant<int, 0>{});
        if (t >= ntot) break;
        step(std::integral_constant<int, 1>{});
        if (t >= ntot) break;
        step(std::integral_constant<int, 2>{});
    }
    // register loads of x past the last step are still in flight
    __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);
    if (nt > 0) {   // y of the last tile
        lds_barrier();
        store_prev_y(*(const lds_u32x4 *)(uintptr_t)y_get);
    }

    if constexpr (MULTI) {
        if (nt == 0) {   // empty sequence: every head's final state is its initial state
            for (int k = 0; k < K; ++k) {
                if (k > 0) load_init(st, k);
                store_final(k);
            }
        } else {
            store_final(K - 1);
        }
    } else {
        float *fd = a.final_states + ((int64_t)(s * H + h) * P + pw + q) * N + nb;
#pragma unroll
        for (int u = 0; u < NTH; ++u) *reinterpret_cast<f32x4 *>(fd + n_of(u)) = st[u];
    }
}
#endif

template <int N>
hipError_t launch_scan_split_instance(const ScanArgs &a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.S * a.H * a.nptiles / a.items;
    if (blocks == 0) return hipSuccess;
    if (a.items > 1)
        hipLaunchKernelGGL((ssd_scan_split_kernel<N, true>), dim3((unsigned)blocks), dim3(SplitShape<N>::kThreads), 0,
                           stream, a, a.chunk_state_dst);
    else
        hipLaunchKernelGGL((ssd_scan_split_kernel<N, false>), dim3((unsigned)blocks), dim3(SplitShape<N>::kThreads), 0,
                           stream, a, a.chunk_state_dst);
    return hipGetLastError();
}

}  // namespace ssd
