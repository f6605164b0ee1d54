// Warp-specialised variant of the fused tile-walk scan, for bf16 inputs with
// dstate 128, headdim a multiple of 64 and chunk_size >= 64 (the Mamba2 layer
// shapes of the prefill workloads).
//
// One workgroup owns one (sequence, head, 64 headdim columns) and walks the
// sequence in 64-token tiles, like the other two scan kernels, but its eight
// waves take two roles:
//   - chain waves 0-3 (one per SIMD): wave c owns headdim columns
//     16 c .. 16 c + 15 and carries their WHOLE 128 x 16 float32 state in
//     registers. Per tile it computes the inter-chunk term Y = C h_in scaled by
//     2^(s_i), the state update h_out = 2^(s_last) h_in + B^T (w o x), and,
//     one tile later, the intra-chunk and D terms Y += M x. No state data ever
//     moves between waves.
//   - helper waves 4-7 (one per SIMD, beside a chain wave): the scan tables of
//     the next tile (softplus of dt + bias, inclusive log2-decay cumsum s_j,
//     2^(s_j), w_j = delta_j 2^(s_last - s_j)) and the decay matrix of the
//     current tile M[i][j] = (C_i . B_j) 2^(s_i - s_j) delta_j (j <= i), + D on
//     the diagonal, on the matrix cores; and the memory pipeline, split by
//     latency class: helpers 4 and 5 fetch the C and the B tiles (direct-to-LDS
//     loads two tiles ahead, mostly L2 hits) and helpers 6 and 7 load x three
//     tiles ahead through registers and store y (HBM). Each waits only for its
//     own loads (vector memory retires in issue order per wave).
//   - The C and B tiles of a (sequence, group) are read by every workgroup of
//     its heads and headdim tiles at about the same time, so each would see the
//     first reader's HBM latency; these workgroups share an L2 prefetch of the
//     tiles four tiles ahead, each touching 8 lines of each tile.
// The only cross-wave dependencies are through LDS buffers that are written
// one tile before they are read, so one barrier per tile suffices and the
// chain and helper waves of a SIMD overlap their matrix, LDS and vector work
// instead of running the same phase in lockstep.
//
// The chunked form is the per-chunk decomposition of the SSD layer (the
// kernel list of the problem statement: chunk cumsum, chunk state, state
// passing, C B^T, chunk scan); a chunk longer than 64 tokens is walked as
// consecutive 64-token tiles with the state carried between them (an exact
// re-association of the recurrence). The decay that reaches the entering
// state at token i is 2^(s_i) with s_i the INCLUSIVE cumsum at i, and the
// total decay of a tile is read at its last valid token (delta = 0 past the
// sequence end keeps s constant there): the initial-state decay rule of the
// varlen bug-fix page ("[Bugfix] Mamba2 SSD varlen bug fix initstates decay",
// Purpose).
//
// Step t (one barrier at its start), buffers indexed mod 3:
//   chain:  M_{t-1} x_{t-1} added to y_{t-1}, y_{t-1} -> X[t-1] (over x_{t-1});
//           x_t^T from X[t]; inter term of tile t from C_t (stage t) and h_{t-1};
//           state update from B_t (stage t), x_t and the tables of tile t;
//           checkpoint of h_t when tile t ends a chunk.
//   helper: C/B of tile t+2 (+ dt of tile t+3) -> stage t+2 (direct loads;
//           in one burst at the start of the step in launches that write
//           checkpoints, else in three parts between the M blocks below),
//           then wait for stage t+1 (helpers 4, 5);
//           y_{t-2} from X[t+1] -> HBM, then x_{t+1} (registers) -> X[t+1];
//           x of tile t+4 -> registers (helpers 6, 7);
//           tables of tile t+1 from its dt (which rode with stage t) -> T[t+1]
//           (helpers 6, 7);
//           blocks of M_t from stage t and T[t] -> M[t] (all four).
// So stage t is read in step t only, X[t] holds x_t in step t and y_t from
// step t+1 to t+2, M_t and the tables are produced one step before their
// readers use them, and every buffer is free again before it is rewritten.
//
// LDS (bytes): 3 stages x (C 16384 + B 16384), 3 x 256 dt, 3 X tiles of 8192
// (64 tokens x 64 columns), 3 M tiles of 8192 (64 x 64 bf16), 3 x 1024 tables,
// 4 x 2048 checkpoint staging, 768 scratch (prefetch targets and the empty dt loads):
// 160,256 in all (one workgroup per CU).
// Layouts (16-byte chunks XOR-swizzled by row). The masks were chosen by
// measurement on this chip (the LDS bank-conflict counter over each access
// pattern of this kernel, replayed alone): a mask that spreads the 16 lanes of
// a quarter-wave over all banks is not enough for 16-byte reads, which the
// hardware serves in an order that also couples quarter-waves.
//   C, B rows (256 bytes): chunk k of row r at k ^ fbc(r mod 16), fbc the
//     row's four bits rotated by one, (r0 r1 r2 r3) -> (r3 r0 r1 r2): both the
//     16-byte row reads and the transposed 8-byte reads of B run at the
//     conflict-free rate (a plain k ^ r costs twice the cycles on the former);
//   x and y rows (128 bytes): chunk k of row r at k ^ swz(r), swz = (r2, r1, r3);
//   decay matrix rows (128 bytes): chunk k at k ^ (r mod 8) (its 16-byte
//     row reads; its 8-byte writes conflict 2-way in every layout tried).
//
// Operand layouts on v_mfma_f32_16x16x32_bf16: lane l = 16 g + q supplies
// row/column q and k slots 8 g .. 8 g + 7 of both operands; any assignment of k
// to slots works when both operands use it. The chain wave's state: lane
// (g, q) holds h[n][p] for p = 16 c + q and n = 32 g + 4 (u ^ (g & 1)) + r in
// register u (0..7), element r; the state update's A operand (B^T, by
// transposed reads) has block u's row 4 m + r at n = 32 m + 4 (u ^ (m & 1)) + r,
// so the accumulator holds exactly that layout, and k step c of the inter term
// takes lane group g's n = 32 g + 8 c .. + 7, i.e. registers 2c, 2c+1 (in
// g-dependent order) as the A operand and one 16-byte read of each C row.
#pragma once

#include "ssd_scan_split.hpp"

namespace ssd {

struct WsShape {
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kCols = 64;                  // headdim columns per workgroup
    static constexpr int kN = 128;                    // dstate
    static constexpr int kRB = kN * 2;                // bytes per B/C row (256)
    static constexpr int kRX = kCols * 2;             // bytes per x / y tile row (128)
    static constexpr int kTileBC = kTile * kRB;       // 16 KB
    static constexpr int kTileX = kTile * kRX;        // 8 KB
    static constexpr int kTileM = kTile * kTile * 2;  // 8 KB
    static constexpr int kTab = 4 * 64;               // S, E, Dl, W
    static constexpr int kStageE = 2048;              // checkpoint staging per chain wave (4 rows x 512 bytes)
    static constexpr int bytes() {
        return 6 * kTileBC + 3 * 256 + 3 * kTileX + 3 * kTileM + 3 * kTab * 4 + 4 * kStageE + 3 * 256;
    }
    // C/B helper: vector memory instructions per step (16 direct 1 KB loads of
    // its tile, one of dt, then the L2 prefetch below); its wait for the stage
    // fetched one step earlier sees that step's prefetch and one whole step
    // after the stage's last load: kBcWait
    static constexpr int kBcPerStep = 18;
    // L2 prefetch of tile f + kPf while tile f is fetched, spread over the
    // workgroups that read the same C and B tiles (the heads of one group and
    // their headdim tiles, up to 16): each touches 4 rows (8 lines) of its
    // helper's tile with one 4-byte direct load into a scratch area, after the
    // stage loads (in the several-heads instances with more rows per
    // workgroup, during the first head only)
    static constexpr int kPf = 4;
    static constexpr int kBcWait = kBcPerStep + 1;
    // x helper: per step 4 y stores, then (after the wait) 4 register loads of
    // x; the loads of tile t + 1 are the last ones of step t - 3, so when step
    // t writes them to LDS two whole steps and this step's stores follow them
    static constexpr int kXStores = 4, kXLoads = 4;
    static constexpr int kWaitX = 2 * (kXStores + kXLoads) + kXStores;
    static_assert(kWaitX <= 63, "vmcnt range");
    // 16-byte chunk swizzles (XOR masks by row): C and B tiles (256-byte rows),
    // x / y tiles and the decay matrix (128-byte rows)
    __device__ static int fbc(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
    __device__ static int swz(int r) { return ((r >> 2) & 1) | (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2); }
    __device__ static int swm(int r) { return r & 7; }
};
static_assert(WsShape::bytes() <= kLdsLimit, "LDS plan");

// The helper wave's pipeline loads. Their buffer resources are rebuilt every
// step from wave-uniform values that the compiler may compute on the vector
// unit and move to SGPRs with v_readfirstlane; a vector memory instruction
// must come at least five wait states after such a write, and one wait state
// must separate the M0 write from a direct-to-LDS load. The compiler pads its
// own code but not these asm statements, so each carries s_nop 4 (five wait
// states) right before its load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int OFF, int STAGE>
__device__ __forceinline__ void ws_dma16(const u32x4 &r0, uint32_t lds_base, int voff) {
    const u32x4 r = sgpr4(r0);
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds ; ssd-stage %4"
                 :: "v"(voff), "s"(r), "s"(lds_base), "i"(OFF), "i"(STAGE) : "memory", "m0", "scc");
}
template <int OFF, int STAGE>
__device__ __forceinline__ void ws_dma4(const u32x4 &r0, uint32_t lds_base, int voff) {
    const u32x4 r = sgpr4(r0);
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds ; ssd-stage %4"
                 :: "v"(voff), "s"(r), "s"(lds_base), "i"(OFF), "i"(STAGE) : "memory", "m0", "scc");
}
// An untracked register load of x (see load16_untracked), non-temporal: x is
// read once, and keeping it out of the caches' retained lines measured 5 %
// faster on the prefix-cache workload.
template <int STAGE>
__device__ __forceinline__ void ws_load16_untracked(u32x4 &dst, const u32x4 &r0, int voff) {
    const u32x4 r = sgpr4(r0);
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2, 0 offen nt ; ssd-stage %3"
                 : "=v"(dst) : "v"(voff), "s"(r), "i"(STAGE) : "memory");
}
// A 16-byte y store through a resource of wave-uniform words (s_nop 1 after
// it: see export_store16). Plain write-back stores: in this kernel they timed
// 3-5 % faster than non-temporal ones, for y and for the checkpoints.
__device__ __forceinline__ void ws_store16(const u32x4 &v, const u32x4 &r0, int off) {
    const u32x4 r = sgpr4(r0);
    asm volatile("s_nop 4\n\tbuffer_store_dwordx4 %0, %1, %2, 0 offen\n\ts_nop 1" :: "v"(v), "v"(off), "s"(r) : "memory");
}
// A 16-byte checkpoint store (plain; see ws_store16 and export_store16)
__device__ __forceinline__ void ws_export_store16(const u32x4 &v, const u32x4 &r, int off) {
    asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen ; ssd-export\n\ts_nop 1" :: "v"(v), "v"(off), "s"(r) : "memory");
}
#pragma clang diagnostic pop

// The decay-matrix blocks (I, J) each helper wave computes: the ten blocks on
// and below the diagonal, 3 + 3 + 2 + 2 (each block is 4 matrix ops).
struct WsBlocks0 { static constexpr int n = 3; __device__ static constexpr int I(int) { return 3; } __device__ static constexpr int J(int k) { return k; } };
struct WsBlocks1 { static constexpr int n = 3; __device__ static constexpr int I(int) { return 2; } __device__ static constexpr int J(int k) { return k; } };
struct WsBlocks2 { static constexpr int n = 2; __device__ static constexpr int I(int k) { return k == 0 ? 3 : 1; } __device__ static constexpr int J(int k) { return k == 0 ? 3 : 0; } };
struct WsBlocks3 { static constexpr int n = 2; __device__ static constexpr int I(int k) { return k == 0 ? 0 : 1; } __device__ static constexpr int J(int k) { return k == 0 ? 0 : 1; } };

// kInterleave: the C/B helpers issue their tile fetch in three parts between
// their decay-matrix blocks (launches without checkpoints: 2-5 % faster there)
// instead of in one burst at the start of the step (launches that write
// checkpoints: the interleaved order timed 4-9 % slower with them).
// kMulti: the workgroup walks a.items consecutive heads of one (sequence,
// group) pair as one stream of a.items x nt tiles (stream index u = k nt + j:
// head h0 + k, tile j). The heads share the sequence's B and C tiles, so the
// C/B fetch restarts at the sequence's first tile with each head, while dt, x
// and y follow the head, and the per-head constants (A, D, dt bias) are read
// from lanes of a register by the head index. The pipeline runs on from one
// head into the next; at a head's last tile the chain waves store its final
// state and load the next head's initial state, whose bf16 operand of the
// inter term is formed in the next step, after the intra term (the load's
// latency overlaps the barrier and that work).
template <int N, bool kInterleave, bool kMulti>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ssd_scan_ws_kernel(ScanArgs a, const int32_t *__restrict__ dstmap)
#if !defined(__HIP_DEVICE_COMPILE__)
{   // the host pass only needs the signature (for the launch stub)
}
#else
{
    static_assert(N == 128, "laid out for dstate 128");
    using O = Ops<uint16_t>;
    using Frag = O::Frag;
    using SH = WsShape;
    constexpr int RB = SH::kRB, RX = SH::kRX, TAB = SH::kTab;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

    __shared__ __align__(16) unsigned char sC[3 * SH::kTileBC];
    __shared__ __align__(16) unsigned char sB[3 * SH::kTileBC];
    __shared__ __align__(16) float sDt[3 * 64];
    __shared__ __align__(16) float sDtNull[3 * 64];   // target of the second C/B helper's empty dt loads
    __shared__ __align__(16) unsigned char sX[3 * SH::kTileX];
    __shared__ __align__(16) unsigned char sM[3 * SH::kTileM];
    __shared__ __align__(16) float tabs[3 * TAB];
    __shared__ __align__(16) unsigned char sE[4 * SH::kStageE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane & 15, g = lane >> 4;

    if (__builtin_nontemporal_load(a.error_flag) & SSD_DATA_BAD_CU_SEQLENS) return;
    int rank, h, pt;
    if constexpr (kMulti) decode_block_multi(a, blockIdx.x, rank, h, pt);   // h: the first head
    else decode_block(a, blockIdx.x, rank, h, pt);
    const int s = a.seq_order[rank];
    if (s < 0 || s >= a.S) return;
    const int grp = h / (a.H / a.G);
    const int H = a.H, P = a.P, G = a.G, cs = a.cs;
    int64_t tb = a.cu_seqlens[s], te = a.cu_seqlens[s + 1];
    tb = tb < 0 ? 0 : (tb > a.T ? a.T : tb);
    te = te < tb ? tb : (te > a.T ? a.T : te);
    const int L = (int)(te - tb);
    const int nt = (L + kTile - 1) / kTile;
    const int tpc = cs / kTile;               // tiles per chunk (cs >= 64, a power of two)
    const int c0 = a.seq_chunk_start[s];
    const int p0 = pt * SH::kCols;
    const int xrow = H * P * 2;               // bytes between tokens of x / y
    const int browg = G * N * 2;              // bytes between tokens of B / C
    auto clamp_len = [](int rem) __attribute__((always_inline)) { return rem < 0 ? 0 : (rem > kTile ? kTile : rem); };
    const bool has_init = a.init != nullptr && (a.has_init == nullptr || a.has_init[s] != 0);
    const int K = kMulti ? a.items : 1;   // heads walked
    const int ntot = K * nt;              // tiles of the stream

    if (wave < 4) {
        // =====================================================================
        // chain wave cw: columns pw .. pw + 15
        // =====================================================================
        const int cw = wave;
        const int pw = p0 + 16 * cw;
        const bool godd = (g & 1) != 0;
        auto n_of = [&](int u) __attribute__((always_inline)) { return 32 * g + 4 * (u ^ (g & 1)); };
        f32x4 st[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) st[u] = f32x4{0, 0, 0, 0};
        const int64_t state_row = ((int64_t)(s * H + h) * P + pw + q) * N;
        const int64_t head_state = (int64_t)P * N;   // between consecutive heads' states
        if (has_init) {
            const float *src = a.init + state_row;
#pragma unroll
            for (int u = 0; u < 8; ++u) st[u] = *reinterpret_cast<const f32x4 *>(src + n_of(u));
        }
        float *fd = a.final_states + state_row;
        if (nt == 0) {
#pragma unroll
            for (int u = 0; u < 8; ++u) *reinterpret_cast<f32x4 *>(fd + n_of(u)) = st[u];
            if constexpr (kMulti) {   // the other heads: final = initial state
                for (int k = 1; k < K; ++k) {
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        st[u] = has_init ? *reinterpret_cast<const f32x4 *>(a.init + state_row + k * head_state + n_of(u))
                                         : f32x4{0, 0, 0, 0};
#pragma unroll
                    for (int u = 0; u < 8; ++u) *reinterpret_cast<f32x4 *>(fd + k * head_state + n_of(u)) = st[u];
                }
            }
            return;
        }

        // bf16 fragments of h_in for the inter term (k step c: n = 32 g + 8 c .. + 7)
        Frag hf[4];
        auto make_hf = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t a0 = pack_bf16(st[2 * c][0], st[2 * c][1]), a1 = pack_bf16(st[2 * c][2], st[2 * c][3]);
                const uint32_t b0 = pack_bf16(st[2 * c + 1][0], st[2 * c + 1][1]),
                               b1 = pack_bf16(st[2 * c + 1][2], st[2 * c + 1][3]);
                hf[c].w = godd ? u32x4{b0, b1, a0, a1} : u32x4{a0, a1, b0, b1};
            }
        };
        make_hf();

        // Per-lane LDS addresses (stage 0 / buffer 0; stages, row blocks and
        // k steps over tokens are immediate offsets).
        //   C rows 16 I + q, chunk 4 g + c (swizzled); B the same + kTileBC
        uint32_t ac[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) ac[c] = lds_addr(sC) + q * RB + 16 * ((4 * g + c) ^ SH::fbc(q));
        //   B^T (transposed reads) of register block u: lane (t4, m) of group g
        //   supplies token row 8 g + t4 (+ 4), n = 32 m + 4 (u ^ (m & 1)) .. + 3
        uint32_t abt[8][2];
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const int r = 8 * g + (q >> 2) + 4 * hi, m = q & 3;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                abt[u][hi] = lds_addr(sB) + r * RB + 16 * ((4 * m + (u >> 1)) ^ SH::fbc(r)) +
                             8 * ((u ^ m) & 1);
        }
        //   x^T (transposed): token row 8 g + t4 (+ 4), columns 16 cw + 4 m .. + 3
        uint32_t axf[2];
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const int r = 8 * g + (q >> 2) + 4 * hi, m = q & 3;
            axf[hi] = lds_addr(sX) + r * RX + 16 * ((2 * cw + (m >> 1)) ^ SH::swz(r)) + 8 * (m & 1);
        }
        //   M rows 16 I + q, chunk 4 ks + g (swizzled)
        uint32_t amr[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) amr[ks] = lds_addr(sM) + q * RX + 16 * ((4 * ks + g) ^ SH::swm(q));
        //   y rows 16 I + q, columns 16 cw + 4 g .. + 3 (8 bytes)
        const uint32_t ayw = lds_addr(sX) + q * RX + 16 * ((2 * cw + (g >> 1)) ^ SH::swz(q)) + 8 * (g & 1);
#pragma unroll
        for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(ac[c]));
#pragma unroll
        for (int u = 0; u < 8; ++u) asm volatile("" : "+v"(abt[u][0]), "+v"(abt[u][1]));

        // checkpoints: the state after tile t is exported when the tile ends a
        // chunk (or is the sequence's last); slots of 64 chunks at a time, lane k
        // holding chunk ex_win + k
        int ex_tile = a.chunk_states != nullptr ? min(tpc, nt) - 1 : nt;
        int ex_chunk = c0, ex_win = c0;
        auto load_slots = [&](int c) __attribute__((always_inline)) {
            const int gc = c + lane;
            return (gc >= 0 && gc < a.max_chunks) ? (dstmap ? dstmap[gc] : gc) : -1;
        };
        int slots = a.chunk_states != nullptr ? load_slots(ex_win) : -1;
        const int slots0 = slots;   // (multi-head: every head restarts at the sequence's first chunk)
        uint64_t ck_base = uni64((uint64_t)(uintptr_t)a.chunk_states + (uint64_t)((h * P + pw) * N) * 4);
        const uint64_t ck_slot = uni64((uint64_t)H * P * N * 4);
        //   staging: 4 state rows x 512 bytes; chunk k of row i at k ^ (k >> 4 | 2 i)
        const uint32_t e_base = lds_addr(sE) + SH::kStageE * cw;
        auto e_pos = [](int i, int k) __attribute__((always_inline)) { return 512 * i + 16 * (k ^ (((k >> 4) & 1) | (2 * i))); };
        auto export_state = [&](int dsl) __attribute__((always_inline)) {
            const u32x4 re = buf_rsrc(ck_base + (uint64_t)dsl * ck_slot, 16 * N * 4);
#pragma unroll
            for (int rnd = 0; rnd < 4; ++rnd) {
                if ((q >> 2) == rnd) {
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        *(lds_u32x4 *)(uintptr_t)(e_base + e_pos(q & 3, n_of(u) / 4)) = __builtin_bit_cast(u32x4, st[u]);
                }
                wave_lds_sync();
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int i = 2 * k + (lane >> 5), kk = lane & 31;
                    const u32x4 v = *(const lds_u32x4 *)(uintptr_t)(e_base + e_pos(i, kk));
                    ws_export_store16(v, re, ((4 * rnd + i) * N) * 4 + 16 * kk);
                }
                wave_lds_sync();
            }
        };

        f32x4 accp[4];   // Y^T of the previous tile (inter term, scaled)
        Frag xtp[2];     // x^T of the previous tile
#pragma unroll
        for (int I = 0; I < 4; ++I) accp[I] = f32x4{0, 0, 0, 0};
        xtp[0].w = xtp[1].w = u32x4{0, 0, 0, 0};
        int jt = 0, kh = 0;   // (multi-head) tile of the step within its head, and the head
        // (multi-head) an L2 prefetch of the next head's initial state two tiles
        // before the hand-over (or at the start of a one-tile head's step): one
        // 4-byte direct load per 128-byte line of the wave's 16 state rows,
        // into a scratch LDS area that no one reads. The register load at the
        // hand-over then waits for L2, not HBM.
        const uint32_t lds_pfc = __builtin_amdgcn_readfirstlane(lds_addr(sDtNull));
        const int go_pfc = (lane >> 2) * N * 4 + 128 * (lane & 3);
        const int64_t wave_state = ((int64_t)(s * H + h) * P + pw) * N;

        auto step = [&](auto slot_c, int t) __attribute__((always_inline)) {
            constexpr int SLOT = decltype(slot_c)::value, PREV = (SLOT + 2) % 3;
            constexpr int OS = SLOT * SH::kTileBC, OX = SLOT * SH::kTileX, OXP = PREV * SH::kTileX,
                          OMP = PREV * SH::kTileM;
            const float *tab = tabs + SLOT * TAB;
            if (t > 0 && t <= ntot) {
                // ---- intra-chunk and D terms of tile t - 1: Y^T += x^T M^T
                Frag mf[4][2];
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        if (ks <= I / 2) mf[I][ks].w = *(const lds_u32x4 *)(uintptr_t)(amr[ks] + OMP + 16 * RX * I);
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        if (ks <= I / 2) accp[I] = O::mma(accp[I], xtp[ks], mf[I][ks]);
                // y of tile t - 1 -> X[PREV] (over its x, which this wave no longer needs)
#pragma unroll
                for (int I = 0; I < 4; ++I)
                    *(lds_u32x2 *)(uintptr_t)(ayw + OXP + 16 * RX * I) =
                        u32x2{pack_bf16(accp[I][0], accp[I][1]), pack_bf16(accp[I][2], accp[I][3])};
            }
            if (t >= ntot) return;
            if constexpr (kMulti) {
                if (has_init && kh + 1 < K && jt == (nt >= 2 ? nt - 2 : 0)) {
                    const u32x4 rp = buf_rsrc(uni64((uint64_t)(uintptr_t)(a.init + wave_state + (kh + 1) * head_state)), 16 * N * 4);
                    ws_dma4<0, 9>(rp, lds_pfc, go_pfc);
                }
            }

            // ---- x^T of tile t (A operand of the intra term, B operand of the state update)
            Frag xt[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) xt[ks] = tr2(axf[0] + OX + 32 * RX * ks, axf[1] + OX + 32 * RX * ks);
            // w_j for the lane's 8 tokens of each k step
            f32x4 wv[2][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    wv[ks][e] = *(const lds_f32x4 *)(uintptr_t)(lds_addr(tab + 192) + 4 * (32 * ks + 8 * g + 4 * e));
            float eic[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) eic[I] = tab[64 + 16 * I + q];
            const float sL = tab[63];

            // ---- inter term: Y^T = h_in^T . C^T, column i scaled by 2^(s_i), and
            // the state update h = 2^(s_last) h + B^T (w o x). The C fragments are
            // read before the first matrix op and the first k step's B^T fragments
            // half-way through the inter term (scheduling barriers keep the
            // compiler from sinking the reads to their uses, which serialises LDS
            // latency into the chain).
            Frag cf[4][4], bt0[8];
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int c = 0; c < 4; ++c) cf[I][c] = rf16(ac[c] + OS + 16 * RB * I);
            if constexpr (kMulti) make_hf();   // (h_in may be a new head's initial state, loaded at the end of the last step)
            __builtin_amdgcn_sched_barrier(0);
            f32x4 acc[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) acc[I] = f32x4{0, 0, 0, 0};
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int I = 0; I < 4; ++I) acc[I] = O::mma(acc[I], hf[c], cf[I][c]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 8; ++u) bt0[u] = tr2(abt[u][0] + OS, abt[u][1] + OS);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = 2; c < 4; ++c)
#pragma unroll
                for (int I = 0; I < 4; ++I) acc[I] = O::mma(acc[I], hf[c], cf[I][c]);
            __builtin_amdgcn_s_setprio(0);
            Frag xw[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float w0 = wv[ks][i >> 1][2 * (i & 1)], w1 = wv[ks][i >> 1][2 * (i & 1) + 1];
                    xw[ks].w[i] = pack_bf16(bf16_lo(xt[ks].w[i]) * w0, bf16_hi(xt[ks].w[i]) * w1);
                }
            }
            const float e = fast_exp2(sL);
#pragma unroll
            for (int u = 0; u < 8; ++u) st[u] *= e;
            Frag bt1[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) bt1[u] = tr2(abt[u][0] + OS + 32 * RB, abt[u][1] + OS + 32 * RB);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int u = 0; u < 8; ++u) st[u] = O::mma(st[u], bt0[u], xw[0]);
#pragma unroll
            for (int u = 0; u < 8; ++u) st[u] = O::mma(st[u], bt1[u], xw[1]);
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int I = 0; I < 4; ++I) acc[I] *= eic[I];
            if constexpr (!kMulti) make_hf();
#pragma unroll
            for (int I = 0; I < 4; ++I) accp[I] = acc[I];
            xtp[0] = xt[0];
            xtp[1] = xt[1];

            // ---- checkpoint of the state after tile t
            if ((kMulti ? jt : t) == ex_tile) {
                if (ex_chunk - ex_win >= 64) {   // next window (once per 64 checkpoints)
                    ex_win = ex_chunk;
                    slots = load_slots(ex_win);
                }
                int dsl = __builtin_amdgcn_readlane(slots, ex_chunk - ex_win);
                if (dsl >= a.capacity) {
                    if (lane == 0) atomicOr(a.error_flag, SSD_DATA_BAD_SLOT);
                    dsl = -1;
                }
                dsl = __builtin_amdgcn_readfirstlane(dsl);
                ++ex_chunk;
                ex_tile = min(ex_tile + tpc, nt - 1);
                if (dsl >= 0) export_state(dsl);
            }
            if constexpr (kMulti) {
                if (++jt == nt) {   // the head's last tile: the next head's initial state in, this head's final state out
                    // (the loads are issued before the stores, so that waiting for
                    // them, vector memory retiring in issue order, does not also
                    // wait for the stores; the operands of the step's products are
                    // dead here, so the loaded state has registers of its own)
                    jt = 0;
                    f32x4 nx[8];
                    if (kh + 1 < K) {
                        const float *src = a.init + state_row + (kh + 1) * head_state;
#pragma unroll
                        for (int u = 0; u < 8; ++u)
                            nx[u] = has_init ? *reinterpret_cast<const f32x4 *>(src + n_of(u)) : f32x4{0, 0, 0, 0};
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) *reinterpret_cast<f32x4 *>(fd + n_of(u)) = st[u];
                    if (++kh < K) {
                        fd += head_state;
                        ck_base += (uint64_t)head_state * 4;
                        ex_tile = a.chunk_states != nullptr ? min(tpc, nt) - 1 : nt;
                        ex_chunk = c0;
                        ex_win = c0;
                        slots = slots0;
#pragma unroll
                        for (int u = 0; u < 8; ++u) st[u] = nx[u];
                    }
                }
            }
        };

        int t = 0;
        while (t < ntot + 2) {
            lds_barrier();
            step(std::integral_constant<int, 0>{}, t);
            if (++t >= ntot + 2) break;
            lds_barrier();
            step(std::integral_constant<int, 1>{}, t);
            if (++t >= ntot + 2) break;
            lds_barrier();
            step(std::integral_constant<int, 2>{}, t);
            ++t;
        }
        if constexpr (!kMulti) {   // (multi-head: stored at each head's last tile)
#pragma unroll
            for (int u = 0; u < 8; ++u) *reinterpret_cast<f32x4 *>(fd + n_of(u)) = st[u];
        }
    } else {
        // =====================================================================
        // helper waves: hw 0, 1 (on the SIMDs of chain waves 0, 1) fetch the C
        // and B tiles; hw 2, 3 load x and store y. Each kind waits only for its
        // own loads: vector memory retires in issue order per wave, so a wave
        // that waited for its C/B stage (L2 latency) behind x loads issued just
        // before it (HBM latency) would couple the two pipelines.
        // =====================================================================
        const int hw = wave - 4;
        if (nt == 0) return;
        __builtin_assume(nt > 0 && nt < (1 << 24));   // (every step loop below runs nt + 2 > 2 times)
        __builtin_assume(ntot >= nt && ntot < (1 << 26));
        float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
        float a2 = a.A[h] * kLog2e;
        float Dh = a.D ? a.D[h] : 0.0f;
        // (multi-head) lane k holds the constants of head h + k; the stream
        // position (head, tile) of the step in us / ut
        float bias_v = 0.0f, a2_v = 0.0f, d_v = 0.0f;
        if constexpr (kMulti) {
            if (lane < K) {
                bias_v = a.dt_bias ? a.dt_bias[h + lane] : 0.0f;
                a2_v = a.A[h + lane] * kLog2e;
                d_v = a.D ? a.D[h + lane] : 0.0f;
            }
        }
        int us = 0, ut = 0;
        // the tile after stream position (k, j)
        auto next_pos = [&](int &k, int &j) __attribute__((always_inline)) {
            const bool w = j + 1 == nt;
            j = w ? 0 : j + 1;
            k = w ? k + 1 : k;
        };
        // constants for the step's work: the tables of the next tile (its head's
        // A and dt bias) and the decay matrix of this tile (its head's D)
        auto step_consts = [&]() __attribute__((always_inline)) {
            if constexpr (kMulti) {
                const int kn = (ut + 1 == nt) ? us + 1 : us;
                const int kc = kn < K ? kn : K - 1;
                bias = readlane(bias_v, kc);
                a2 = readlane(a2_v, kc);
                Dh = readlane(d_v, us < K ? us : K - 1);
            }
        };

        // zero the blocks above the diagonal that the intra term reads (M rows
        // 0..15 x columns 16..31 and rows 32..47 x columns 48..63), all buffers
        {
            const int i = 32 * (lane >> 5) + (lane & 15), J = 1 + 2 * (lane >> 5), half = (lane >> 4) & 1;
            if (hw < 3) {
                const uint32_t p = lds_addr(sM) + hw * SH::kTileM + i * RX + 16 * ((2 * J + half) ^ SH::swm(i));
                *(lds_u32x4 *)(uintptr_t)p = u32x4{0, 0, 0, 0};
            }
        }
        // scan tables of a tile from delta (lane j = token j, 0 past the end),
        // written by the x helpers from one prefix sum each: hw 2 S = s_j and
        // Dl = delta_j, hw 3 E = 2^(s_j) and W = delta_j 2^(s_last - s_j). (The
        // C/B helpers, the last to reach the barrier, compute none: one table
        // per helper timed 2-5 % slower.)
        auto tables = [&](float *tab, float d) __attribute__((always_inline)) {
            const float v = wave_scan(d * a2);
            if (hw == 2) {
                tab[lane] = v;
                tab[128 + lane] = d;
            } else {
                tab[64 + lane] = fast_exp2(v);
                tab[192 + lane] = d * fast_exp2(readlane(v, 63) - v);
            }
        };
        {
            float d = 0.0f;
            if (lane < clamp_len(L)) d = softplus_hw(a.dt[(tb + lane) * H + h] + bias);
            if (hw >= 2) tables(tabs, d);
        }
        // Decay-matrix blocks (I, J), J <= I: D[j][i] = B_j . C_i over n, then
        // M[i][j] = D 2^(s_i - s_j) delta_j (0 for j > i) + D_h [i == j].
        // Lane (g, q): i = 16 I + q, j = 16 J + 4 g + r.
        uint32_t ahc[4], ahb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            ahc[c] = lds_addr(sC) + q * RB + 16 * ((4 * g + c) ^ SH::fbc(q));
            ahb[c] = lds_addr(sB) + q * RB + 16 * ((4 * g + c) ^ SH::fbc(q));
        }
        const uint32_t amw = lds_addr(sM) + q * RX + 8 * (g & 1);
        auto mblocks = [&](auto slot_c, auto blocks_c) __attribute__((always_inline)) {
            constexpr int SLOT = decltype(slot_c)::value;
            constexpr int OS = SLOT * SH::kTileBC;
            const float *tab = tabs + SLOT * TAB;
            using BL = decltype(blocks_c);
            static_for<BL::n>([&](auto b_c) {
                constexpr int I = BL::I(decltype(b_c)::value), J = BL::J(decltype(b_c)::value);
                Frag cf[4], bf[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    cf[c] = rf16(ahc[c] + OS + 16 * RB * I);
                    bf[c] = rf16(ahb[c] + OS + 16 * RB * J);
                }
                f32x4 d = {0, 0, 0, 0};
#pragma unroll
                for (int c = 0; c < 4; ++c) d = O::mma(d, bf[c], cf[c]);
                const int i = 16 * I + q;
                const float si = tab[i];
                const f32x4 sj = *(const lds_f32x4 *)(uintptr_t)(lds_addr(tab) + 4 * (16 * J + 4 * g));
                const f32x4 dj = *(const lds_f32x4 *)(uintptr_t)(lds_addr(tab + 128) + 4 * (16 * J + 4 * g));
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * J + 4 * g + r;
                    float f = fast_exp2(si - sj[r]) * dj[r];
                    if constexpr (I == J) f = j <= i ? f : 0.0f;
                    v[r] = d[r] * f;
                    if constexpr (I == J) v[r] += j == i ? Dh : 0.0f;
                }
                *(lds_u32x2 *)(uintptr_t)(amw + SLOT * SH::kTileM + 16 * RX * I + 16 * ((2 * J + (g >> 1)) ^ SH::swm(q))) =
                    u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
            });
        };
        // the compute of step t common to both kinds: tables of tile t + 1
        // (from the dt that rode with stage t) and this helper's blocks of M_t
        auto compute = [&](auto slot_c, int t) __attribute__((always_inline)) {
            constexpr int SLOT = decltype(slot_c)::value, NEXT = (SLOT + 1) % 3;
            if (hw >= 2 && t + 1 < ntot) {   // tables of tile t + 1
                const int jn = kMulti ? ((ut + 1 == nt) ? 0 : ut + 1) : t + 1;
                const int Ln = clamp_len(L - jn * kTile);
                tables(tabs + NEXT * TAB, softplus_hw(sDt[SLOT * 64 + lane] + bias + (lane < Ln ? 0.0f : -INFINITY)));
            }
            if (t < ntot) {     // decay matrix of tile t
                if (hw == 0) mblocks(slot_c, WsBlocks0{});
                else if (hw == 1) mblocks(slot_c, WsBlocks1{});
                else if (hw == 2) mblocks(slot_c, WsBlocks2{});
                else mblocks(slot_c, WsBlocks3{});
            }
        };

        // The interleaved form: a block's fragment reads and its math as
        // separate calls, so that the caller can place its memory instructions
        // in between.
        auto mread = [&](auto slot_c, auto blocks_c, auto b_c, Frag (&cf)[3][4], Frag (&bf)[3][4]) __attribute__((always_inline)) {
            constexpr int OS = decltype(slot_c)::value * SH::kTileBC;
            using BL = decltype(blocks_c);
            constexpr int Bk = decltype(b_c)::value;
            if constexpr (Bk < BL::n) {
                constexpr int I = BL::I(Bk), J = BL::J(Bk);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    cf[Bk][c] = rf16(ahc[c] + OS + 16 * RB * I);
                    bf[Bk][c] = rf16(ahb[c] + OS + 16 * RB * J);
                }
            }
        };
        auto mmath = [&](auto slot_c, auto blocks_c, auto b_c, const Frag (&cf)[3][4], const Frag (&bf)[3][4]) __attribute__((always_inline)) {
            constexpr int SLOT = decltype(slot_c)::value;
            using BL = decltype(blocks_c);
            constexpr int Bk = decltype(b_c)::value;
            if constexpr (Bk < BL::n) {
                constexpr int I = BL::I(Bk), J = BL::J(Bk);
                const float *tab = tabs + SLOT * TAB;
                f32x4 d = {0, 0, 0, 0};
#pragma unroll
                for (int c = 0; c < 4; ++c) d = O::mma(d, bf[Bk][c], cf[Bk][c]);
                const int i = 16 * I + q;
                const float si = tab[i];
                const f32x4 sj = *(const lds_f32x4 *)(uintptr_t)(lds_addr(tab) + 4 * (16 * J + 4 * g));
                const f32x4 dj = *(const lds_f32x4 *)(uintptr_t)(lds_addr(tab + 128) + 4 * (16 * J + 4 * g));
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * J + 4 * g + r;
                    float f = fast_exp2(si - sj[r]) * dj[r];
                    if constexpr (I == J) f = j <= i ? f : 0.0f;
                    v[r] = d[r] * f;
                    if constexpr (I == J) v[r] += j == i ? Dh : 0.0f;
                }
                *(lds_u32x2 *)(uintptr_t)(amw + SLOT * SH::kTileM + 16 * RX * I + 16 * ((2 * J + (g >> 1)) ^ SH::swm(q))) =
                    u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
            }
        };
        using B0c = std::integral_constant<int, 0>;
        using B1c = std::integral_constant<int, 1>;
        using B2c = std::integral_constant<int, 2>;
        auto next_tables = [&](auto slot_c, int t) __attribute__((always_inline)) {   // tables of tile t + 1
            constexpr int SLOT = decltype(slot_c)::value, NEXT = (SLOT + 1) % 3;
            if (hw >= 2 && t + 1 < ntot) {
                const int jn = kMulti ? ((ut + 1 == nt) ? 0 : ut + 1) : t + 1;
                const int Ln = clamp_len(L - jn * kTile);
                tables(tabs + NEXT * TAB, softplus_hw(sDt[SLOT * 64 + lane] + bias + (lane < Ln ? 0.0f : -INFINITY)));
            }
        };

        if (hw < 2) {
            // ---- C/B helper: hw 0 fetches the C tiles, hw 1 the B tiles (16
            // direct 1 KB loads each), hw 0 also the dt of the tile after (hw 1
            // an empty load in its place), and each one 4-byte L2 prefetch:
            // 18 vector memory instructions per step.
            // Block b of a tile: lane l -> row 4 b + l / 16, LDS chunk l mod 16
            // <- global chunk (l mod 16) ^ fbc(row)
            int go[16];
#pragma unroll
            for (int b = 0; b < 16; ++b) {
                const int r = 4 * b + (lane >> 4);
                go[b] = r * browg + 16 * ((lane & 15) ^ SH::fbc(r & 15));
            }
            const int go_d = lane * H * 4;
            auto rfl = [](uint32_t v) __attribute__((always_inline)) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); };
            // (only hw 0 loads the tile's dt; hw 1 issues the same instruction
            // with an empty range into a scratch area, keeping the counts equal)
            const uint32_t lds_t = rfl(hw == 0 ? lds_addr(sC) : lds_addr(sB)),
                           lds_dt = rfl(hw == 0 ? lds_addr(sDt) : lds_addr(sDtNull));
            const void *src = hw == 0 ? a.C : a.B;
            u32x4 r_t = buf_rsrc(uni64((uint64_t)(uintptr_t)src + (uint64_t)((tb * G + grp) * N) * 2), 0);
            u32x4 r_d = buf_rsrc(uni64((uint64_t)(uintptr_t)a.dt + (uint64_t)((tb + kTile) * H + h) * 4), 0);
            int f_rem = L;   // tokens from the tile being fetched on
            const uint32_t step_bc = (uint32_t)__builtin_amdgcn_readfirstlane(kTile * browg),
                           step_d = (uint32_t)__builtin_amdgcn_readfirstlane(kTile * H * 4);
            auto advance = [](u32x4 &r, uint32_t inc) __attribute__((always_inline)) {
                const uint64_t v = (((uint64_t)r.y) << 32 | r.x) + inc;
                r.x = (uint32_t)v;
                r.y = (uint32_t)(v >> 32);
            };
            int go_pf;
            if constexpr (kMulti) {   // H / G / K x nptiles workgroups share a tile: 64 / that rows each (at least 4)
                const int nsh = (H / G / K) * a.nptiles, rps = nsh >= 16 ? 4 : 64 / nsh;
                const int pk = ((h % (H / G)) / K) * a.nptiles + pt;
                go_pf = (lane < 2 * rps && rps * pk < 64) ? (rps * pk + (lane >> 1)) * browg + 128 * (lane & 1) : kOob;
            } else {
                const int pk = (h % (H / G)) * a.nptiles + pt;   // this workgroup's share of the prefetch
                go_pf = (lane < 8 && pk < 16) ? (4 * pk + (lane >> 1)) * browg + 128 * (lane & 1) : kOob;
            }
            const uint32_t lds_pfz = rfl(lds_addr(sDtNull) + 256 * hw);
            // (multi-head) stream position of the tile being fetched, and the
            // resources of that fetch: the sequence's C/B rows of its tile, the
            // dt of the tile after (its head's column), and the L2 prefetch
            // (during the first head only: the later heads find the tiles in L2)
            int kf = 0, jf = 0;
            u32x4 r_pfm = r_t;
            auto multi_rsrc = [&]() __attribute__((always_inline)) {
                const uint64_t t_base = (uint64_t)(uintptr_t)src + (uint64_t)((tb * G + grp) * N) * 2;
                const uint64_t d_base = (uint64_t)(uintptr_t)a.dt + (uint64_t)(tb * H + h) * 4;
                r_t = buf_rsrc(uni64(t_base + (uint64_t)jf * step_bc), kf < K ? clamp_len(L - jf * kTile) * browg : 0);
                int kd = kf, jd = jf;
                next_pos(kd, jd);
                r_d = buf_rsrc(uni64(d_base + ((uint64_t)jd * kTile * H + kd) * 4),
                               (hw == 0 && kd < K) ? clamp_len(L - jd * kTile) * H * 4 : 0);
                const int jp = jf + SH::kPf;
                r_pfm = buf_rsrc(uni64(t_base + (uint64_t)jp * step_bc),
                                 (kf == 0 && jp < nt) ? clamp_len(L - jp * kTile) * browg : 0);
            };
            auto fetch = [&](auto slot_c) __attribute__((always_inline)) {
                constexpr int SLOT = decltype(slot_c)::value;
                if constexpr (kMulti) {
                    multi_rsrc();
                } else {
                    r_t.z = (uint32_t)(clamp_len(f_rem) * browg);
                    r_d.z = hw == 0 ? (uint32_t)(clamp_len(f_rem - kTile) * H * 4) : 0u;
                }
                static_for<16>([&](auto b_c) {
                    constexpr int Bk = decltype(b_c)::value;
                    ws_dma16<SLOT * SH::kTileBC + 1024 * Bk, SLOT>(r_t, lds_t, go[Bk]);
                });
                ws_dma4<SLOT * 256, SLOT>(r_d, lds_dt, go_d);
                if constexpr (kMulti) {
                    ws_dma4<0, 9>(r_pfm, lds_pfz, go_pf);
                    next_pos(kf, jf);
                } else {
                    u32x4 r_pf = r_t;
                    advance(r_pf, SH::kPf * step_bc);
                    r_pf.z = (uint32_t)(clamp_len(f_rem - SH::kPf * kTile) * browg);
                    ws_dma4<0, 9>(r_pf, lds_pfz, go_pf);
                    advance(r_t, step_bc); advance(r_d, step_d);
                    f_rem -= kTile;
                }
            };
            // the same fetch in three parts (blocks 0-5, 6-11, 12-15 with dt and
            // the prefetch), placed between the decay-matrix blocks' math
            auto fetch_part = [&](auto slot_c, auto part_c) __attribute__((always_inline)) {
                constexpr int SLOT = decltype(slot_c)::value, PART = decltype(part_c)::value;
                constexpr int B0 = PART * 6, B1 = PART == 2 ? 16 : B0 + 6;
                if constexpr (PART == 0) {
                    if constexpr (kMulti) multi_rsrc();
                    else r_t.z = (uint32_t)(clamp_len(f_rem) * browg);
                }
                static_for<B1 - B0>([&](auto b_c) {
                    constexpr int Bk = B0 + decltype(b_c)::value;
                    ws_dma16<SLOT * SH::kTileBC + 1024 * Bk, SLOT>(r_t, lds_t, go[Bk]);
                });
                if constexpr (PART == 2 && kMulti) {
                    ws_dma4<SLOT * 256, SLOT>(r_d, lds_dt, go_d);
                    ws_dma4<0, 9>(r_pfm, lds_pfz, go_pf);
                    next_pos(kf, jf);
                } else if constexpr (PART == 2) {
                    r_d.z = hw == 0 ? (uint32_t)(clamp_len(f_rem - kTile) * H * 4) : 0u;
                    ws_dma4<SLOT * 256, SLOT>(r_d, lds_dt, go_d);
                    u32x4 r_pf = r_t;
                    advance(r_pf, SH::kPf * step_bc);
                    r_pf.z = (uint32_t)(clamp_len(f_rem - SH::kPf * kTile) * browg);
                    ws_dma4<0, 9>(r_pf, lds_pfz, go_pf);
                    advance(r_t, step_bc); advance(r_d, step_d);
                    f_rem -= kTile;
                }
            };
            fetch(std::integral_constant<int, 0>{});   // tile 0
            fetch(std::integral_constant<int, 1>{});   // tile 1
            wait_vm_stage<SH::kBcWait, 0>();

            // interleaved step t: the C/B of tile t + 2 (+ dt of tile t + 3) in
            // three parts between this helper's blocks of M_t (also computed
            // past the last tile, into a buffer no one reads)
            auto step_blocks = [&](auto slot_c, auto blocks_c) __attribute__((always_inline)) {
                constexpr int FETCH = (decltype(slot_c)::value + 2) % 3;
                using FS = std::integral_constant<int, FETCH>;
                Frag cf[3][4], bf[3][4];
                mread(slot_c, blocks_c, B0c{}, cf, bf);
                fetch_part(FS{}, B0c{});
                mmath(slot_c, blocks_c, B0c{}, cf, bf);
                mread(slot_c, blocks_c, B1c{}, cf, bf);
                fetch_part(FS{}, B1c{});
                mmath(slot_c, blocks_c, B1c{}, cf, bf);
                mread(slot_c, blocks_c, B2c{}, cf, bf);
                fetch_part(FS{}, B2c{});
                mmath(slot_c, blocks_c, B2c{}, cf, bf);
            };
            auto step = [&](auto slot_c, int t) __attribute__((always_inline)) {
                constexpr int SLOT = decltype(slot_c)::value, NEXT = (SLOT + 1) % 3, FETCH = (SLOT + 2) % 3;
                step_consts();
                // (the C/B helpers, the last to reach the barrier, issue at the
                // chain waves' raised priority during their step work: 1-2 %
                // faster on the three bf16 workloads; the x helpers raised too,
                // or these above the chain waves, timed no better)
                __builtin_amdgcn_s_setprio(1);
                if constexpr (kInterleave) {
                    if (hw == 0) step_blocks(slot_c, WsBlocks0{});
                    else step_blocks(slot_c, WsBlocks1{});
                    next_tables(slot_c, t);
                } else {
                    fetch(std::integral_constant<int, FETCH>{});            // tile t + 2
                    compute(slot_c, t);
                }
                __builtin_amdgcn_s_setprio(0);
                wait_vm_stage<SH::kBcWait, NEXT>();                         // stage t + 1 landed
                if constexpr (kMulti) next_pos(us, ut);
            };
            int t = 0;
            while (t < ntot + 2) {
                lds_barrier();
                step(std::integral_constant<int, 0>{}, t);
                if (++t >= ntot + 2) break;
                lds_barrier();
                step(std::integral_constant<int, 1>{}, t);
                if (++t >= ntot + 2) break;
                lds_barrier();
                step(std::integral_constant<int, 2>{}, t);
                ++t;
            }
            __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);
        } else {
            // ---- x helper xh: token rows 32 xh .. 32 xh + 31 of every x and y
            // tile (four 1 KB loads or stores each), x three tiles ahead through
            // registers: 8 vector memory instructions per step.
            // Row r = 32 xh + 8 k + l / 8: LDS chunk l mod 8 <- global chunk (l mod 8) ^ swz(r)
            const int xh = hw - 2;
            int go_x[4], yo[4];
            uint32_t lx[4], ly[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = 32 * xh + 8 * k + (lane >> 3);
                go_x[k] = r * xrow + 16 * ((lane & 7) ^ SH::swz(r));
                yo[k] = r * xrow + 16 * (lane & 7);
                lx[k] = lds_addr(sX) + r * RX + 16 * (lane & 7);
                ly[k] = lds_addr(sX) + r * RX + 16 * ((lane & 7) ^ SH::swz(r));
            }
            const uint64_t x_seq = uni64((uint64_t)(uintptr_t)a.x + (uint64_t)((tb * H + h) * P + p0) * 2);
            const uint64_t y_seq = uni64((uint64_t)(uintptr_t)a.y + (uint64_t)((tb * H + h) * P + p0) * 2);
            const uint32_t step_x = (uint32_t)__builtin_amdgcn_readfirstlane(kTile * xrow);
            {   // x of tile 0 straight into X[0]
                const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(uintptr_t)x_seq, 0, __builtin_amdgcn_readfirstlane(clamp_len(L) * xrow), kBufFlags);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    *(lds_u32x4 *)(uintptr_t)lx[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, go_x[k], 0, 0));
            }
            __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);   // nothing outstanding before the pipeline starts
            u32x4 xr[3][4];
            int xg_t = 1;
            // (multi-head) stream positions of the next x tile to load and of the
            // next y tile to store; advanced with selects only (no control flow
            // may separate an untracked load from its wait)
            int kx = 0, jx = 0, ky = 0, jy = 0;
            if constexpr (kMulti) next_pos(kx, jx);   // tile 1
            const uint32_t head_x = (uint32_t)(P * 2);   // bytes between consecutive heads' columns
            auto xload = [&](auto set_c) __attribute__((always_inline)) {   // x of tile xg_t into register set SET
                constexpr int SET = decltype(set_c)::value;
                if constexpr (kMulti) {
                    const u32x4 r = buf_rsrc(x_seq + (uint64_t)kx * head_x + (uint64_t)jx * step_x,
                                             kx < K ? clamp_len(L - jx * kTile) * xrow : 0);
#pragma unroll
                    for (int k = 0; k < 4; ++k) ws_load16_untracked<3 + SET>(xr[SET][k], r, go_x[k]);
                    next_pos(kx, jx);
                } else {
                    const u32x4 r = buf_rsrc(x_seq + (uint64_t)xg_t * step_x, clamp_len(L - xg_t * kTile) * xrow);
#pragma unroll
                    for (int k = 0; k < 4; ++k) ws_load16_untracked<3 + SET>(xr[SET][k], r, go_x[k]);
                }
                ++xg_t;
            };
            auto ystore = [&](auto slot_c, int yt) __attribute__((always_inline)) {   // y of tile yt from X[SLOT] (zero-sized range if no tile)
                constexpr int SLOT = decltype(slot_c)::value;
                u32x4 r;
                if constexpr (kMulti) {
                    const int len = (yt >= 0 && yt < ntot) ? clamp_len(L - jy * kTile) : 0;
                    r = buf_rsrc(y_seq + (uint64_t)ky * head_x + (uint64_t)jy * step_x, len * xrow);
                    int k2 = ky, j2 = jy;
                    next_pos(k2, j2);
                    ky = yt >= 0 ? k2 : ky;
                    jy = yt >= 0 ? j2 : jy;
                } else {
                    const int len = (yt >= 0 && yt < nt) ? clamp_len(L - yt * kTile) : 0;
                    r = buf_rsrc(y_seq + (uint64_t)(yt < 0 ? 0 : yt) * step_x, len * xrow);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const u32x4 v = *(const lds_u32x4 *)(uintptr_t)(ly[k] + SLOT * SH::kTileX);
                    ws_store16(v, r, yo[k]);
                }
            };
            const u32x4 r_null = buf_rsrc(y_seq, 0);
            // prologue: three steps' worth of vector memory instructions (x of tiles 1..3)
            static_for<3>([&](auto k_c) {
                constexpr int K = decltype(k_c)::value;
#pragma unroll
                for (int i = 0; i < SH::kXStores; ++i) null_store16(r_null);
                xload(std::integral_constant<int, (K + 1) % 3>{});   // tile K + 1
            });

            auto step = [&](auto slot_c, int t) __attribute__((always_inline)) {
                constexpr int SLOT = decltype(slot_c)::value, NEXT = (SLOT + 1) % 3;
                step_consts();
                ystore(std::integral_constant<int, NEXT>{}, t - 2);    // y of tile t - 2 (in X[t + 1])
                wait_vm_stage<SH::kWaitX, 3 + NEXT>();                  // x of tile t + 1
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    reg_fence(xr[NEXT][k]);
                    *(lds_u32x4 *)(uintptr_t)(lx[k] + NEXT * SH::kTileX) = xr[NEXT][k];
                }
                xload(std::integral_constant<int, NEXT>{});             // tile t + 4
                // (the multi-head instances always take this form: with the
                // four-way block choice of compute() the compiler fails on them)
                if constexpr (kInterleave || kMulti) {
                    next_tables(slot_c, t);
                    if (t < ntot) {   // this helper's blocks of M_t, one at a time
                        Frag cf[3][4], bf[3][4];
                        if (hw == 2) {
                            mread(slot_c, WsBlocks2{}, B0c{}, cf, bf); mmath(slot_c, WsBlocks2{}, B0c{}, cf, bf);
                            mread(slot_c, WsBlocks2{}, B1c{}, cf, bf); mmath(slot_c, WsBlocks2{}, B1c{}, cf, bf);
                        } else {
                            mread(slot_c, WsBlocks3{}, B0c{}, cf, bf); mmath(slot_c, WsBlocks3{}, B0c{}, cf, bf);
                            mread(slot_c, WsBlocks3{}, B1c{}, cf, bf); mmath(slot_c, WsBlocks3{}, B1c{}, cf, bf);
                        }
                    }
                } else {
                    compute(slot_c, t);
                }
                if constexpr (kMulti) next_pos(us, ut);
            };
            int t = 0;
            while (t < ntot + 2) {
                lds_barrier();
                step(std::integral_constant<int, 0>{}, t);
                if (++t >= ntot + 2) break;
                lds_barrier();
                step(std::integral_constant<int, 1>{}, t);
                if (++t >= ntot + 2) break;
                lds_barrier();
                step(std::integral_constant<int, 2>{}, t);
                ++t;
            }
            // register loads of x past the last tile are still in flight
            __builtin_amdgcn_s_waitcnt(WaitVm<0>::imm);
        }
    }
}
#endif

template <int N>
hipError_t launch_scan_ws_instance(const ScanArgs &a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.S * a.H * a.nptiles / a.items;
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), wg(WsShape::kThreads);
    const bool ex = a.chunk_states != nullptr;
    if (a.items > 1) {
        if (ex) hipLaunchKernelGGL((ssd_scan_ws_kernel<N, false, true>), grid, wg, 0, stream, a, a.chunk_state_dst);
        else hipLaunchKernelGGL((ssd_scan_ws_kernel<N, true, true>), grid, wg, 0, stream, a, a.chunk_state_dst);
    } else {
        if (ex) hipLaunchKernelGGL((ssd_scan_ws_kernel<N, false, false>), grid, wg, 0, stream, a, a.chunk_state_dst);
        else hipLaunchKernelGGL((ssd_scan_ws_kernel<N, true, false>), grid, wg, 0, stream, a, a.chunk_state_dst);
    }
    return hipGetLastError();
}

}  // namespace ssd
