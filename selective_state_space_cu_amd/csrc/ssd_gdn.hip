// Chunked gated delta rule (the GDN layers' recurrent state, whose chunk
// kernel the prefix-caching page extends with a per-chunk intermediate-state
// export; chunk size 64) for gfx950: bf16 q, k, v, o; float32 gates, betas and
// states.
//
// Recurrence (per sequence and value head h, key head g = h / (H/G); state S
// value-major, dv x dk):
//     S_t = e^(gate_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = scale S_t q_t.
// Chunked form (exact re-association; WY representation): within a chunk with
// entering state S0 (H0 = S0^T, dk x dv), inclusive log-gate cumsum G_i and
// gamma_i = e^(G_i):
//     A_ij = beta_i e^(G_i - G_j) k_i . k_j   (j < i),   T = (I + A)^-1 (unit lower triangular)
//     W = T diag(beta gamma) K,   U = T diag(beta) V - W H0          (the chunk's write values)
//       = T (diag(beta) V - diag(beta gamma) K H0)                   (the form computed here)
//     O = scale (diag(gamma) Q H0 + (e^(G_i - G_j) q_i . k_j)_{j <= i} U)
//     H_next = gamma_last H0 + K^T diag(e^(G_last - G)) U
// (U_i is the delta-rule write value of token i; the token loop computes the
// same map one token at a time.)
//
// Two kernels on one stream:
//  ssd_gdn_prep_kernel, persistent workgroups (four per CU) over the (chunk,
//    key head) items, whose value heads share the K K^T sub-tiles:
//    A on the matrix cores (bf16 K K^T, masked by the decay, float32), T by
//    forward substitution on the four 16 x 16 diagonal blocks and block merges
//    on the float32 matrix cores
//        T_IJ = -T_II (sum_K A_IK T_KJ)   (first the blocks next to the diagonal,
//                                         then the 32 x 32 corner),
//    written to the workspace as bf16 (64 x 64 per chunk and head). T depends
//    on neither the state nor the values, so no chunk waits for another here.
//  ssd_gdn_scan_kernel, one workgroup per (sequence, value head, 64 value
//    columns), walks the chunks in order with the state in registers, split by
//    keys over two waves per SIMD; per chunk only matrix-core products: K H0,
//    Q H0, the causal Q K^T (masked), U = T (beta V - beta gamma K H0), O and the
//    state update, with two barriers. The next chunk's K, Q, V and T are loaded
//    into registers while the current chunk computes.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssd_scan.hpp"

namespace ssd {

namespace {

constexpr int kGdnDk = 128;            // key dimension
constexpr int kGdnCols = 64;           // value columns per scan workgroup
constexpr int kGdnChunk = 64;          // tokens per chunk
// Row tiles (K, Q, W: 64 rows of 128 bf16): rows in groups of 8 (pitch kPB, 128
// extra bytes per group), and within every 32-column k step the columns
// interleaved in groups of 4 -- c = 32 kc + 16 hh + 4 gg + x sits at
// 32 kc + 8 gg + 4 hh + x -- so that the eight elements lane group gg feeds the
// matrix cores in one k step (columns 4 gg.. and 16 + 4 gg..) are one 16-byte read,
// and any 4 consecutive columns from a multiple of 4 stay 8 contiguous bytes
// (the transposed reads).
constexpr int kPB = kGdnDk * 2 + 32, kGB = 8 * kPB + 128, kTileR = 8 * kGB;
// V and U rows (64 value columns): pitch 144; T and Mq rows: pitch 160
[[maybe_unused]] constexpr int kPX = kGdnCols * 2 + 16, kTileV = kGdnChunk * kPX;
[[maybe_unused]] constexpr int kMPB = (kGdnChunk + 16) * 2, kTileM = kGdnChunk * kMPB;
// float32 16 x 16 blocks of the lower triangle of a 64 x 64 matrix, stored
// compactly: block (I, J), I >= J, at (I (I + 1) / 2 + J) * kBlk floats, rows of
// kBP floats (16-byte aligned)
constexpr int kBP = 20, kBlk = 16 * kBP, kTri = 10 * kBlk;
static_assert(2 * kTri * 4 >= kTileR, "T and T^T blocks reuse the K tile");
static_assert(kGdnWsBytes == kGdnChunk * kGdnChunk * 2, "workspace: one bf16 T per (chunk, head)");

[[maybe_unused]] __device__ __forceinline__ int rt_row(int r) { return (r >> 3) * kGB + (r & 7) * kPB; }
[[maybe_unused]] __device__ __forceinline__ int rt_col(int c) {   // byte offset of column c in a row
    return (32 * (c >> 5) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3)) * 2;
}
// row fragment of k step kc for lane group g (the permuted k order of the state fragments)
[[maybe_unused]] __device__ __forceinline__ Ops<uint16_t>::Frag rt_frag(const unsigned char *tile, int row, int kc,
                                                                        int g) {
    return Ops<uint16_t>::Frag{*reinterpret_cast<const u32x4 *>(tile + rt_row(row) + 64 * kc + 16 * g)};
}
// transposed fragment: column c0 + q of rows kb .. kb + 7 (kb a multiple of 8)
[[maybe_unused]] __device__ __forceinline__ Ops<uint16_t>::Frag rt_tr(const unsigned char *tile, int kb, int c0,
                                                                      int q) {
    using O = Ops<uint16_t>;
    return O::tr(tile + rt_row(kb) + O::tr_row(q) * kPB + rt_col(c0 + O::tr_col(q)), 4 * kPB);
}
// one staged 16-byte piece (columns 8 cpos .. 8 cpos + 7 of row r) into a row tile
[[maybe_unused]] __device__ __forceinline__ void rt_store(unsigned char *tile, int r, int cpos, const u32x4 &v) {
    unsigned char *row = tile + rt_row(r);
    *reinterpret_cast<u32x2 *>(row + rt_col(8 * cpos)) = u32x2{v[0], v[1]};
    *reinterpret_cast<u32x2 *>(row + rt_col(8 * cpos + 4)) = u32x2{v[2], v[3]};
}
// compiler fence: LDS reads issued above it stay above (batched ahead of their products)
[[maybe_unused]] __device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }
// XCD-aware work order: workgroup b runs on XCD b mod 8, each XCD with its own
// L2. Items that read the same key-head data (R of them per key head) are put
// 8 apart in b, on one XCD, so that their q and k rows come from one L2; plain
// order when the grid does not split evenly. Returns (key-head item, sharer).
[[maybe_unused]] __device__ __forceinline__ int2 xcd_order(int b, int nblocks, int R) {
    if (R <= 1 || nblocks % (8 * R) != 0) return int2{b / R, b % R};
    const int r = b >> 3;
    return int2{(r / R) * 8 + (b & 7), r % R};
}
[[maybe_unused]] __device__ __forceinline__ int tri_blk(int I, int J) { return (I * (I + 1) / 2 + J) * kBlk; }

[[maybe_unused]] __device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// 16 x 16 x 16 float32 product on the matrix cores. Lane (g, q) supplies
// a[r] = X[q][4 g + r] and b[r] = Y[4 g + r][q] (step r sums k = 4 g + r over
// the four lane groups); the result holds (X Y)[4 g + r][q] in element r, which
// is the b operand layout of the next product.
[[maybe_unused]] __device__ __forceinline__ f32x4 mm16(const f32x4 &a, const f32x4 &b, f32x4 c) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c = mfma4(a[r], b[r], c);
    return c;
}

// Buffer resource over `bytes` bytes from p (loads past them read zero)
[[maybe_unused]] __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, kBufFlags);
}
// 16-byte pieces of a chunk's q or k rows (64 rows x 16 pieces, 4 per thread;
// rows past the chunk's Lc >= 1 tokens read zero)
[[maybe_unused]] __device__ __forceinline__ void load_rows(u32x4 (&kv)[4], const uint16_t *base, int64_t t0, int Lc,
                                                           int G, int grp, int tid) {
    const int rowb = G * kGdnDk * 2;
    const __amdgpu_buffer_rsrc_t r = rsrc(base + (t0 * G + grp) * kGdnDk, (int64_t)(Lc - 1) * rowb + 256);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int piece = tid + 256 * i;
        kv[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (piece >> 4) * rowb + 16 * (piece & 15), 0, 0);
    }
}
// one lane per token of a chunk: x[(t0 + lane) H + h] (zero past the chunk's Lc >= 1 tokens)
[[maybe_unused]] __device__ __forceinline__ float load_token(const float *x, int64_t t0, int Lc, int H, int h,
                                                             int lane) {
    const __amdgpu_buffer_rsrc_t r = rsrc(x + t0 * H + h, (int64_t)(Lc - 1) * H * 4 + 4);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, lane * H * 4, 0, 0));
}

// The three sub-tiles (I, J), I >= J, of the lower triangle of a 64 x 64 matrix
// that role r (0..3) computes: ten over four roles, roles 2 and 3 repeat their
// last sub-tile (identical writes)
[[maybe_unused]] __device__ __forceinline__ int sub_tile(int r, int n) {
    const uint32_t codes = r == 0 ? 0x333000u : r == 1 ? 0x311110u : r == 2 ? 0x212120u : 0x333222u;
    return (codes >> (8 * n)) & 0xff;   // I in the high nibble, J in the low
}

}  // namespace

// ---------------------------------------------------------------------------
// T = (I + A)^-1 for every (chunk, value head)
// ---------------------------------------------------------------------------
//
// Persistent workgroups of four waves; item = (chunk, key head, block of up to
// four of its value heads), taken in steps of the grid. The item's k rows and
// their Gram sub-tiles K K^T are shared by its value heads, which differ only
// in beta and the gates: per value head, A from the Gram sub-tiles held in
// registers, then T. The next item's k rows, gates and betas are loaded into
// registers while the current one computes (wave w: value head w of the block),
// and nothing waits for them before the next item begins.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4)))
void ssd_gdn_prep_kernel(GdnArgs a)
#if !defined(__HIP_DEVICE_COMPILE__)
{
}
#else
{
    using O = Ops<uint16_t>;
    constexpr int CH = kGdnChunk, kHB = 4;   // value heads per item (at most)
    __shared__ __align__(16) float fTT[2 * kTri];    // K rows (row tile) first; then T and T^T blocks
    __shared__ __align__(16) float fA[kTri];         // A blocks (float32, strictly lower)
    __shared__ __align__(16) float tab[kHB * 2 * 64]; // per value head of the item: G (log2), beta
    unsigned char *const sK = reinterpret_cast<unsigned char *>(fTT);
    float *const fT = fTT, *const fTt = fTT + kTri;   // T_IJ blocks; (T_IJ)^T blocks

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane & 15, g = lane >> 4;
    // the waves' roles in the phases below rotate between workgroups, so that the
    // longer roles of the workgroups on one CU fall on different SIMDs
    const int role = (wave + (int)(blockIdx.x >> 8)) & 3;

    if (__builtin_nontemporal_load(a.error_flag) & SSD_DATA_BAD_CU_SEQLENS) return;
    const int H = a.H, G = a.G, R = H / G;
    const int nblk = (R + kHB - 1) / kHB;            // value-head blocks per key head
    const int nitems = a.max_chunks * G * nblk;
    // an item's chunk, token range, first value head and value-head count; false for a
    // chunk that holds no tokens
    struct Item { int gc, t0, Lc, h0, nh; };
    auto span = [&](int it, Item &m) -> bool {
        m.gc = it / (G * nblk);
        const int rest = it - m.gc * (G * nblk), grp = rest / nblk, blk = rest - grp * nblk;
        m.h0 = grp * R + kHB * blk;
        m.nh = min(kHB, R - kHB * blk);
        // read through the constant address space (scalar loads): vector loads here would
        // make the item's first wait also wait for the previous item's stores
        typedef const __attribute__((address_space(4))) int cint;
        const int sq = ((cint *)(uintptr_t)a.chunk_seq_idx)[m.gc];
        if (sq < 0 || sq >= a.S) return false;
        const int c0 = ((cint *)(uintptr_t)a.chunk_offsets)[m.gc], c1 = ((cint *)(uintptr_t)a.chunk_offsets)[m.gc + 1];
        if (c0 < 0 || c1 > a.T || c1 <= c0 || c1 - c0 > CH) return false;
        m.t0 = c0;
        m.Lc = c1 - c0;
        return true;
    };
    u32x4 kv[4];                  // the item's k rows, 4 pieces of 16 bytes per thread
    float gt = 0.0f, bt = 0.0f;   // wave w: gate and beta of the item's value head w (lane = token)
    // issued on every path, with empty buffer ranges (reads of zero) where there is
    // nothing to load, so that no register copy has to wait for these loads
    auto prefetch = [&](const Item &m, bool valid) {
        const int rowb = G * kGdnDk * 2;
        const __amdgpu_buffer_rsrc_t rk =
            rsrc(a.k + ((int64_t)m.t0 * G + m.h0 / R) * kGdnDk, valid ? (int64_t)(m.Lc - 1) * rowb + 256 : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int piece = tid + 256 * i;
            kv[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (piece >> 4) * rowb + 16 * (piece & 15), 0, 0);
        }
        const bool head = valid && wave < m.nh;
        const int64_t tok = (int64_t)m.t0 * H + m.h0 + (head ? wave : 0);
        const int64_t tb = head ? (int64_t)(m.Lc - 1) * H * 4 + 4 : 0;
        gt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(a.gate + tok, tb), lane * H * 4, 0, 0));
        bt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(a.beta + tok, tb), lane * H * 4, 0, 0));
    };

    int item = blockIdx.x;
    Item cur = {0, 0, 0, 0, 0};
    bool ok = item < nitems && span(item, cur);
    prefetch(cur, ok);
    while (item < nitems) {
        const int nxt = item + (int)gridDim.x;
        Item nx = {0, 0, 0, 0, 0};
        const bool okn = nxt < nitems && span(nxt, nx);
        f32x4 kk[3];
        if (ok) {
            lds_barrier();   // the previous item's reads of its tables and of its last T are done
#pragma unroll
            for (int i = 0; i < 4; ++i) rt_store(sK, (tid + 256 * i) >> 4, (tid + 256 * i) & 15, kv[i]);
            if (wave < cur.nh) {   // inclusive cumsum of the log2-decay (zero past the chunk: neutral)
                tab[wave * 128 + lane] = wave_scan(gt * kLog2e);
                tab[wave * 128 + 64 + lane] = bt;
            }
            lds_barrier();

            // ---- Gram sub-tiles kk[m][x] = k_i . k_j of the role's sub-tiles (I, J), I >= J;
            //      lane (g, q): i = 16 I + q, j = 16 J + 4 g + x
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int code = sub_tile(role, m), I = code >> 4, J = code & 15;
                kk[m] = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    kk[m] = O::mma(kk[m], rt_frag(sK, 16 * J + q, kc, g), rt_frag(sK, 16 * I + q, kc, g));
            }
        }
        prefetch(nx, okn);   // the next item's loads fly while this one computes
        if (ok) {
            for (int r = 0; r < cur.nh; ++r) {
                const float *const tG = tab + r * 128, *const tBeta = tG + 64;
                // ---- A sub-tiles: A[i][j] = beta_i e^(G_i - G_j) k_i . k_j (j < i)
#pragma unroll
                for (int m = 0; m < 3; ++m) {
                    const int code = sub_tile(role, m), I = code >> 4, J = code & 15;
                    const int i = 16 * I + q;
                    const float gi = tG[i], bi = tBeta[i];
                    const f32x4 gj = *reinterpret_cast<const f32x4 *>(tG + 16 * J + 4 * g);
                    f32x4 fa;
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const float e = fast_exp2(fminf(gi - gj[x], 0.0f));
                        fa[x] = (16 * J + 4 * g + x < i) ? bi * kk[m][x] * e : 0.0f;
                    }
                    *reinterpret_cast<f32x4 *>(fA + tri_blk(I, J) + q * kBP + 4 * g) = fa;
                }
                lds_barrier();

                // ---- diagonal blocks by forward substitution, all four by the wave of role 0 (lane
                //      group g: block g; lane column j = q): T[i][j] = [i == j] - sum_{m < i} A[i][m] T[m][j]
                if (role == 0) {
                    const float *ab = fA + tri_blk(g, g);
                    float tc[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) tc[i] = i == q ? 1.0f : 0.0f;
                    // columns of A in pairs, each read as 8-byte row pieces just before its two
                    // steps (a fence before each pair keeps the reads from all being issued up
                    // front, which would take more registers than there are)
                    float2 ar[16];
#pragma unroll
                    for (int m = 0; m < 15; ++m) {
                        if ((m & 1) == 0) {
                            lds_fence();
#pragma unroll
                            for (int i = m + 1; i < 16; ++i) ar[i] = *reinterpret_cast<const float2 *>(ab + i * kBP + m);
                        }
#pragma unroll
                        for (int i = m + 1; i < 16; ++i) tc[i] = fmaf(-((m & 1) ? ar[i].y : ar[i].x), tc[m], tc[i]);
                    }
                    float *tb = fT + tri_blk(g, g), *tt = fTt + tri_blk(g, g);
#pragma unroll
                    for (int i = 0; i < 16; ++i) tb[i * kBP + q] = tc[i];
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4)
                        *reinterpret_cast<f32x4 *>(tt + q * kBP + 4 * i4) =
                            f32x4{tc[4 * i4], tc[4 * i4 + 1], tc[4 * i4 + 2], tc[4 * i4 + 3]};
                }
                lds_barrier();

                // ---- blocks next to the diagonal: T_10 (role 0), T_32 (role 1): T_{J+1,J} = -T_{J+1,J+1} A_{J+1,J} T_JJ
                if (role < 2) {
                    const int J = 2 * role, I = J + 1;
                    const f32x4 p = mm16(*reinterpret_cast<const f32x4 *>(fA + tri_blk(I, J) + q * kBP + 4 * g),
                                         *reinterpret_cast<const f32x4 *>(fTt + tri_blk(J, J) + q * kBP + 4 * g),
                                         f32x4{0, 0, 0, 0});
                    const f32x4 t = -mm16(*reinterpret_cast<const f32x4 *>(fT + tri_blk(I, I) + q * kBP + 4 * g), p,
                                          f32x4{0, 0, 0, 0});
                    // t[x] = T[16 I + 4 g + x][16 J + q]
#pragma unroll
                    for (int x = 0; x < 4; ++x) fT[tri_blk(I, J) + (4 * g + x) * kBP + q] = t[x];
                    *reinterpret_cast<f32x4 *>(fTt + tri_blk(I, J) + q * kBP + 4 * g) = t;
                }
                lds_barrier();

                // ---- the 32 x 32 corner, one block per role ((2,0), (2,1), (3,0), (3,1)):
                //      Y_KJ = sum_{J <= L <= 1} A_KL T_LJ,  T_IJ = -sum_{2 <= K <= I} T_IK Y_KJ
                {
                    const int I = 2 + (role >> 1), J = role & 1;
                    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
                    for (int K = 2; K < 4; ++K) {
                        if (K > I) continue;
                        f32x4 y = {0, 0, 0, 0};
#pragma unroll
                        for (int L = 0; L < 2; ++L) {
                            if (L < J) continue;
                            y = mm16(*reinterpret_cast<const f32x4 *>(fA + tri_blk(K, L) + q * kBP + 4 * g),
                                     *reinterpret_cast<const f32x4 *>(fTt + tri_blk(L, J) + q * kBP + 4 * g), y);
                        }
                        acc = mm16(*reinterpret_cast<const f32x4 *>(fT + tri_blk(I, K) + q * kBP + 4 * g), y, acc);
                    }
#pragma unroll
                    for (int x = 0; x < 4; ++x) fT[tri_blk(I, J) + (4 * g + x) * kBP + q] = -acc[x];
                }
                lds_barrier();

                // ---- T (unit lower triangular) -> bf16, row-major 64 x 64, into the workspace
                {
                    uint16_t *ws = a.workspace + ((int64_t)cur.gc * H + cur.h0 + r) * (CH * CH);
#pragma unroll
                    for (int it = 0; it < 2; ++it) {
                        const int e = 8 * (tid + 256 * it), i = e >> 6, j0 = e & 63, I = i >> 4, J = j0 >> 4;
                        const float *src = fT + tri_blk(I, J <= I ? J : I) + (i & 15) * kBP + (j0 & 15);
                        const f32x4 lo = *reinterpret_cast<const f32x4 *>(src), hi = *reinterpret_cast<const f32x4 *>(src + 4);
                        float v8[8];
#pragma unroll
                        for (int x = 0; x < 8; ++x) v8[x] = j0 + x <= i ? (x < 4 ? lo[x] : hi[x - 4]) : 0.0f;
                        *reinterpret_cast<u32x4 *>(ws + e) = u32x4{pack_bf16(v8[0], v8[1]), pack_bf16(v8[2], v8[3]),
                                                                   pack_bf16(v8[4], v8[5]), pack_bf16(v8[6], v8[7])};
                    }
                }
            }
        }
        item = nxt;
        cur = nx;
        ok = okn;
    }
}
#endif

// ---------------------------------------------------------------------------
// The chunk walk of one (sequence, value head, 64 value columns)
// ---------------------------------------------------------------------------
//
// Eight waves, two per SIMD: wave w = (vb, kh), vb = w mod 4, kh = w / 4, owns
// value columns 16 vb .. 16 vb + 15 of the slice and keys 64 kh .. 64 kh + 63
// of their state rows (float32, in the accumulator layout of the state update:
// st[u][r] = S[16 vb + q][64 kh + 16 u + 4 g + r] for lane (g, q)), carried
// from chunk to chunk. Per chunk:
//   (1) Mq = (e^(G_i - G_j) q_i . k_j)_{j <= i} (bf16 sub-tiles over the waves),
//       and in registers the wave's key half of K H0 and of Q H0, and its
//       share of U: T applied to beta V on tokens 32 kh .. 32 kh + 31 (zero on
//       the others) minus beta gamma times its key half of K H0;
//       the next chunk's loads in flight;
//   (2) the two key halves' shares of U and of Q H0 are added through LDS
//       (one barrier); U stays in registers in the accumulator
//       layout (token 16 d + 4 g + r, column q), which is the operand layout of
//       both remaining products once their other operand is read in the same
//       token order (32 ks + 4 g + r, then 32 ks + 16 + 4 g + r):
//       O = scale (diag(gamma) Q H0 + Mq U) for the wave's half of the rows,
//       H = gamma_last H + K^T (rho U) for its key half; the state after the
//       chunk to its checkpoint slot;
//   (3) the next chunk's tiles into LDS and its tables (K and the tables into
//       their second buffers), then one barrier: two per chunk.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ssd_gdn_scan_kernel(GdnArgs a)
#if !defined(__HIP_DEVICE_COMPILE__)
{
}
#else
{
    using O = Ops<uint16_t>;
    using Frag = O::Frag;
    constexpr int DK = kGdnDk, CH = kGdnChunk;

    // K and the tables are double-buffered: the next chunk's are staged while this
    // chunk's state update still reads its own
    __shared__ __align__(16) unsigned char sK[2 * kTileR];
    __shared__ __align__(16) unsigned char sQ[kTileR];
    __shared__ __align__(16) unsigned char sV[kTileV];
    __shared__ __align__(16) unsigned char sT[kTileM];
    __shared__ __align__(16) unsigned char sMq[kTileM];
    // exchange between the two key halves: U partials (4 row blocks) and Q H0
    // partials (the 2 row blocks the partner outputs), 16 bytes per lane each
    __shared__ __align__(16) f32x4 xU[8 * 4 * 64];
    __shared__ __align__(16) f32x4 xO[8 * 2 * 64];
    // tables of the chunk: G (log2), gamma, beta, beta gamma, rho (64 each)
    constexpr int kTab = 5 * 64;
    __shared__ __align__(16) float tab[2 * kTab];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int vb = wave & 3, kh = wave >> 2;
    const int q = lane & 15, g = lane >> 4;

    if (__builtin_nontemporal_load(a.error_flag) & SSD_DATA_BAD_CU_SEQLENS) return;
    const int H = a.H, G = a.G, DV = a.dv;
    // (sequence, key head) items; the value heads of one key head and their
    // column slices share its q and k rows
    const int2 it = xcd_order(blockIdx.x, gridDim.x, (H / G) * a.nptiles);
    const int rank = it.x / G, grp = it.x - (it.x / G) * G;
    const int h = grp * (H / G) + it.y / a.nptiles, pt = it.y - (it.y / a.nptiles) * a.nptiles;
    const int s = a.seq_order[rank];
    if (s < 0 || s >= a.S) return;
    int64_t tb = a.cu_seqlens[s], te = a.cu_seqlens[s + 1];
    tb = tb < 0 ? 0 : (tb > a.T ? a.T : tb);
    te = te < tb ? tb : (te > a.T ? a.T : te);
    const int L = (int)(te - tb);
    const int nch = (L + CH - 1) / CH;
    const int c0 = a.seq_chunk_start[s];
    const int v0 = pt * kGdnCols;              // first value column of the workgroup
    const int vw = v0 + 16 * vb;               // first value column of this wave
    const int k0 = 64 * kh;                    // first key of this wave

    // st[u][r] = S[vw + q][k0 + 16 u + 4 g + r]
    f32x4 st[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) st[u] = f32x4{0, 0, 0, 0};
    if (a.init != nullptr && (a.has_init == nullptr || a.has_init[s] != 0)) {
        const float *src = a.init + ((int64_t)(s * H + h) * DV + vw + q) * DK + k0;
#pragma unroll
        for (int u = 0; u < 4; ++u) st[u] = *reinterpret_cast<const f32x4 *>(src + 16 * u + 4 * g);
    }
    // the state loads complete here: left pending into the chunk loop, the
    // compiler's wait before the state's first use inside the loop would also
    // wait for every chunk's prefetch loads issued just before it
    __builtin_amdgcn_s_waitcnt(0);

    // the strictly-upper sub-tiles that the causal products read (row block 0 x
    // column block 1, row block 2 x column block 3) stay zero in Mq
    if (tid < 256) {
        const int t2 = tid & 127, r = t2 >> 3, part = t2 & 7;   // 16 rows x 8 pieces of 4 bytes per sub-tile
        const int I = (tid >> 7) ? 2 : 0, row = 16 * I + r, col = 16 * (I + 1) + 2 * part;
        *reinterpret_cast<uint32_t *>(sMq + row * kMPB + col * 2) = 0u;
    }

    // ---- staging of one chunk: global loads into registers, then LDS
    u32x4 rk[2], rq[2], rv, rt;
    float rgate = 0.0f, rbeta = 0.0f;
    int next_dst = -1;
    const int vrow = H * DV * 2, krow = G * DK * 2;
    // (issued in two parts, so that the issue of the loads is spread over the chunk's work)
    auto stage_load = [&](int c) {
        const int64_t t0 = tb + (int64_t)c * CH;
        const int Lc = min(CH, L - c * CH);
        const __amdgpu_buffer_rsrc_t rK = rsrc(a.k + (t0 * G + grp) * DK, (int64_t)(Lc - 1) * krow + 256);
        const __amdgpu_buffer_rsrc_t rQ = rsrc(a.q + (t0 * G + grp) * DK, (int64_t)(Lc - 1) * krow + 256);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int piece = tid + 512 * i, off = (piece >> 4) * krow + 16 * (piece & 15);
            rk[i] = __builtin_amdgcn_raw_buffer_load_b128(rK, off, 0, 0);
            rq[i] = __builtin_amdgcn_raw_buffer_load_b128(rQ, off, 0, 0);
        }
    };
    auto stage_load2 = [&](int c) {
        const int64_t t0 = tb + (int64_t)c * CH;
        const int Lc = min(CH, L - c * CH);
        const __amdgpu_buffer_rsrc_t rV = rsrc(a.v + (t0 * H + h) * DV + v0, (int64_t)(Lc - 1) * vrow + 128);
        rv = __builtin_amdgcn_raw_buffer_load_b128(rV, (tid >> 3) * vrow + 16 * (tid & 7), 0, 0);
        rt = *reinterpret_cast<const u32x4 *>(a.workspace + ((int64_t)(c0 + c) * H + h) * (CH * CH) + 8 * tid);
        if (wave == 0) {
            rgate = load_token(a.gate, t0, Lc, H, h, lane);
            rbeta = load_token(a.beta, t0, Lc, H, h, lane);
        }
        // checkpoint slot of the chunk (-1: none), kept in a vector register until
        // it is used so that nothing waits for this load before then; loaded
        // unconditionally (an empty buffer range reads zero) so that no path
        // leaves it pending
        const int gc = c0 + c;
        const bool in_grid = a.chunk_states != nullptr && gc >= 0 && gc < a.max_chunks;
        const bool table = in_grid && a.chunk_state_dst != nullptr;
        const int slot = (int)__builtin_amdgcn_raw_buffer_load_b32(
            rsrc(table ? a.chunk_state_dst + gc : a.chunk_state_dst, table ? 4 : 0), 0, 0, 0);
        next_dst = table ? slot : (in_grid ? gc : -1);
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int piece = tid + 512 * i;
            rt_store(sK + buf * kTileR, piece >> 4, piece & 15, rk[i]);
            rt_store(sQ, piece >> 4, piece & 15, rq[i]);
        }
        *reinterpret_cast<u32x4 *>(sV + (tid >> 3) * kPX + 16 * (tid & 7)) = rv;
        *reinterpret_cast<u32x4 *>(sT + (tid >> 3) * kMPB + 16 * (tid & 7)) = rt;
        if (wave == 0) {   // tables G, gamma, beta, beta gamma, rho (lane j = token j; neutral past the end)
            float *const tb = tab + buf * kTab;
            const float v = wave_scan(rgate * kLog2e);   // inclusive cumsum (log2)
            const float gam = fast_exp2(v);
            tb[lane] = v;
            tb[64 + lane] = gam;
            tb[128 + lane] = rbeta;
            tb[192 + lane] = rbeta * gam;
            tb[256 + lane] = fast_exp2(readlane(v, 63) - v);
        }
    };

    int cur_dst = -1;
    if (nch > 0) {
        stage_load(0);
        stage_load2(0);
        stage_store(0);
        cur_dst = next_dst;
    }
    lds_barrier();

    const float scale = a.scale;
    // the chunk loop, one copy per key half (kh is wave-uniform): the choices between the
    // halves' row blocks and token ranges are then made at compile time, not by selects
    auto walk = [&](auto khc) {
        constexpr int kh = decltype(khc)::value;   // (shadows the run-time value)
        constexpr int k0 = 64 * kh;
        for (int c = 0; c < nch; ++c) {
            const int64_t t0 = tb + (int64_t)c * CH;
            const int Lc = min(CH, L - c * CH);
            // the next chunk's tiles (the last chunk stages itself again: every
            // iteration takes the same path, so no load is left pending on a path
            // the compiler's waits must cover)
            const int cn = c + 1 < nch ? c + 1 : c;
            stage_load(cn);
            const int cb = c & 1;   // this chunk's K and table buffers
            const unsigned char *const cK = sK + cb * kTileR;
            const float *const tG = tab + cb * kTab, *const tGam = tG + 64, *const tBeta = tG + 128,
                        *const tBG = tG + 192, *const tRho = tG + 256;

            // ---- (1) Mq sub-tiles (I, J), I >= J, ten over the eight waves (waves 0 and 1 take two);
            //      lane (g, q): i = 16 I + q, j = 16 J + 4 g + r. Fragments are read in batches
            //      ahead of their products (the fences keep the reads together).
    #pragma unroll
            for (int n = 0; n < 2; ++n) {
                if (n == 1 && wave >= 2) break;
                const int code = n == 0 ? (int)((0x3130222120111000ull >> (8 * wave)) & 0xff) : 0x32 + wave;
                const int I = code >> 4, J = code & 15;
                Frag kf[4], qf[4];
    #pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    kf[kc] = rt_frag(cK, 16 * J + q, kc, g);
                    qf[kc] = rt_frag(sQ, 16 * I + q, kc, g);
                }
                const int i = 16 * I + q;
                const float gi = tG[i];
                const f32x4 gj = *reinterpret_cast<const f32x4 *>(tG + 16 * J + 4 * g);
                lds_fence();
                f32x4 qk = {0, 0, 0, 0};
    #pragma unroll
                for (int kc = 0; kc < 4; ++kc) qk = O::mma(qk, kf[kc], qf[kc]);
                float fq[4];
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = fast_exp2(fminf(gi - gj[r], 0.0f));
                    fq[r] = (16 * J + 4 * g + r <= i) ? qk[r] * e : 0.0f;
                }
                O::mstore4(sMq + i * kMPB + (16 * J + 4 * g) * 2, fq);
            }
            // U = T (diag(beta) V - diag(beta gamma) K H0) (W = T diag(beta gamma) K is never formed):
            // this wave's key half of K H0 (token 16 d + 4 g + r, column q) and of Q H0 (token 16 d + q,
            // column 4 g + r); then its share of U, with the beta V term of k step ks = kh, for all four
            // row blocks: U is linear in the key halves, whose shares meet through LDS
            Frag hf[2];   // H0 fragments of this wave's key half: k step kc covers keys k0 + 32 kc .. (permuted)
    #pragma unroll
            for (int kc = 0; kc < 2; ++kc) hf[kc] = O::from_f32(st[2 * kc], st[2 * kc + 1]);
            f32x4 o1[4], uu[4];
            {
                Frag kf[4][2], qf[4][2];
    #pragma unroll
                for (int d = 0; d < 4; ++d)
    #pragma unroll
                    for (int kc = 0; kc < 2; ++kc) {
                        kf[d][kc] = rt_frag(cK, 16 * d + q, 2 * kh + kc, g);
                        qf[d][kc] = rt_frag(sQ, 16 * d + q, 2 * kh + kc, g);
                    }
                lds_fence();
                f32x4 pk[4];
    #pragma unroll
                for (int d = 0; d < 4; ++d) {
                    pk[d] = f32x4{0, 0, 0, 0};
                    o1[d] = f32x4{0, 0, 0, 0};
    #pragma unroll
                    for (int kc = 0; kc < 2; ++kc) {
                        pk[d] = O::mma(pk[d], kf[d][kc], hf[kc]);
                        o1[d] = O::mma(o1[d], hf[kc], qf[d][kc]);
                    }
                }
                // the right operand of T (.) for k step ks, in the token order of the accumulator
                // layout (32 ks + 4 g + r in slots 0-3, 32 ks + 16 + 4 g + r in slots 4-7); T rows are
                // read in the same order
                Frag tf[4][2];
    #pragma unroll
                for (int d = 0; d < 4; ++d)
    #pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        if (ks <= d / 2) tf[d][ks] = O::rowk_perm(sT + (16 * d + q) * kMPB + (32 * ks + 4 * g) * 2);
                const Frag vf = O::tr(sV + (32 * kh + 4 * g + O::tr_row(q)) * kPX + (16 * vb + O::tr_col(q)) * 2, 16 * kPX);
                f32x4 bg[2][2], be[2];
    #pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    bg[ks][0] = *reinterpret_cast<const f32x4 *>(tBG + 32 * ks + 4 * g);
                    bg[ks][1] = *reinterpret_cast<const f32x4 *>(tBG + 32 * ks + 16 + 4 * g);
                }
                be[0] = *reinterpret_cast<const f32x4 *>(tBeta + 32 * kh + 4 * g);
                be[1] = *reinterpret_cast<const f32x4 *>(tBeta + 32 * kh + 16 + 4 * g);
                lds_fence();
                f32x4 bv[2];   // beta V of k step kh (slots 0-3, 4-7)
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t w = vf.w[r >> 1];
                    bv[0][r] = be[0][r] * ((r & 1) ? bf16_hi(w) : bf16_lo(w));
                    const uint32_t w2 = vf.w[2 + (r >> 1)];
                    bv[1][r] = be[1][r] * ((r & 1) ? bf16_hi(w2) : bf16_lo(w2));
                }
                Frag xf[2];
    #pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bool own = ks == kh;
                    f32x4 lo, hi;
    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        lo[r] = (own ? bv[0][r] : 0.0f) - bg[ks][0][r] * pk[2 * ks][r];
                        hi[r] = (own ? bv[1][r] : 0.0f) - bg[ks][1][r] * pk[2 * ks + 1][r];
                    }
                    xf[ks] = O::from_f32(lo, hi);
                }
    #pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uu[d] = f32x4{0, 0, 0, 0};
    #pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        if (ks <= d / 2) uu[d] = O::mma(uu[d], tf[d][ks], xf[ks]);
                }
            }
            stage_load2(cn);
    #pragma unroll
            for (int d = 0; d < 4; ++d) xU[(wave * 4 + d) * 64 + lane] = uu[d];
    #pragma unroll
            for (int dd = 0; dd < 2; ++dd) xO[(wave * 2 + dd) * 64 + lane] = kh ? o1[3 * dd] : o1[1 + dd];
            lds_barrier();
            const int partner = wave ^ 4;
            {
                // fragments of the remaining products, read in the token order of the U fragments
                // (32 ks + 4 g + r in slots 0-3, 32 ks + 16 + 4 g + r in slots 4-7)
                Frag mf[2][2], ktr[4][2];
                f32x4 xu[4], xo[2], r0[2], r1[2];
    #pragma unroll
                for (int d = 0; d < 4; ++d) xu[d] = xU[(partner * 4 + d) * 64 + lane];
    #pragma unroll
                for (int dd = 0; dd < 2; ++dd) {
                    xo[dd] = xO[(partner * 2 + dd) * 64 + lane];
    #pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        mf[dd][ks] = O::rowk_perm(sMq + (16 * (kh ? 1 + dd : 3 * dd) + q) * kMPB + (32 * ks + 4 * g) * 2);
                }
    #pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    r0[ks] = *reinterpret_cast<const f32x4 *>(tRho + 32 * ks + 4 * g);
                    r1[ks] = *reinterpret_cast<const f32x4 *>(tRho + 32 * ks + 16 + 4 * g);
    #pragma unroll
                    for (int u = 0; u < 4; ++u)
                        ktr[u][ks] = O::tr(cK + rt_row(32 * ks + 4 * g) + O::tr_row(q) * kPB + rt_col(k0 + 16 * u + O::tr_col(q)),
                                           2 * kGB);
                }
                const f32x4 gam = {tGam[16 * (kh ? 1 : 0) + q], tGam[16 * (kh ? 2 : 3) + q], 0.0f, 0.0f};
                const float gl = tGam[63];
                lds_fence();
    #pragma unroll
                for (int d = 0; d < 4; ++d) uu[d] += xu[d];
                Frag uf[2], ru[2];
    #pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    uf[ks] = O::from_f32(uu[2 * ks], uu[2 * ks + 1]);
                    ru[ks] = O::from_f32(uu[2 * ks] * r0[ks], uu[2 * ks + 1] * r1[ks]);
                }
                // O rows of this key half (d = 0, 3 or 1, 2): O[token 16 d + q][column 4 g + r]
                const __amdgpu_buffer_rsrc_t ro = rsrc(a.o + (t0 * H + h) * DV + vw, (int64_t)(Lc - 1) * vrow + 32);
    #pragma unroll
                for (int dd = 0; dd < 2; ++dd) {
                    const int d = kh ? 1 + dd : 3 * dd;
                    f32x4 o2 = {0, 0, 0, 0};
    #pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        if (ks == 0 || dd == 1) o2 = O::mma(o2, uf[ks], mf[dd][ks]);
                    const f32x4 oq = (kh ? o1[1 + dd] : o1[3 * dd]) + xo[dd];
                    const float gi = gam[dd];
                    // rows past the chunk fall outside the buffer range and are dropped
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2{pack_bf16(scale * fmaf(oq[0], gi, o2[0]), scale * fmaf(oq[1], gi, o2[1])),
                              pack_bf16(scale * fmaf(oq[2], gi, o2[2]), scale * fmaf(oq[3], gi, o2[3]))},
                        ro, (16 * d + q) * vrow + 8 * g, 0, 0);
                }
                // state update of this key half: st[u] = gamma_last st[u] + K^T (rho U)
    #pragma unroll
                for (int u = 0; u < 4; ++u) {
                    st[u] *= gl;
    #pragma unroll
                    for (int ks = 0; ks < 2; ++ks) st[u] = O::mma(st[u], ktr[u][ks], ru[ks]);
                }
            }
            // the state after the chunk into its checkpoint slot
            if (__builtin_amdgcn_readfirstlane(cur_dst) >= 0) {
                if (__builtin_amdgcn_readfirstlane(cur_dst) >= a.capacity) {
                    if (tid == 0) atomicOr(a.error_flag, SSD_DATA_BAD_SLOT);
                } else {
                    float *dst = a.chunk_states + ((int64_t)__builtin_amdgcn_readfirstlane(cur_dst) * H + h) * DV * DK +
                                 (int64_t)(vw + q) * DK + k0;
    #pragma unroll
                    for (int u = 0; u < 4; ++u) *reinterpret_cast<f32x4 *>(dst + 16 * u + 4 * g) = st[u];
                }
            }

            // ---- (3) the next chunk's K and tables into the other buffers, its Q, V and T over
            //      this chunk's (no wave reads those past the first barrier); one barrier then
            //      makes them visible and orders this chunk's Mq reads before the next chunk's writes
            stage_store(cb ^ 1);
            cur_dst = next_dst;
            lds_barrier();
        }
    };
    if (kh) walk(std::integral_constant<int, 1>{});
    else walk(std::integral_constant<int, 0>{});

    float *fd = a.final_states + ((int64_t)(s * H + h) * DV + vw + q) * DK + k0;
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<f32x4 *>(fd + 16 * u + 4 * g) = st[u];
}
#endif

// Workspace of the allocation-free entry point: one file-scope array, of which
// every GPU the library runs on holds its own copy until the process ends. In
// host code `scratch` only names the symbol; its device address (per device)
// comes from hipGetSymbolAddress, resolved on the first call on each device.
static __device__ __align__(256) unsigned char scratch[kGdnScratchBytes];

hipError_t gdn_scratch(void **ptr) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_gdn(const GdnArgs &a, hipStream_t stream) {
    const int64_t items = (int64_t)a.max_chunks * a.G * ((a.H / a.G + 3) / 4);
    if (items > 0 && a.T > 0) {
        // four workgroups per CU, the items spread evenly over the rounds
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        const int64_t slots = 4 * (int64_t)(cus > 0 ? cus : 1);
        const int64_t rounds = (items + slots - 1) / slots;
        const int64_t grid = (items + rounds - 1) / rounds;
        hipLaunchKernelGGL(ssd_gdn_prep_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t blocks = (int64_t)a.S * a.H * a.nptiles;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(ssd_gdn_scan_kernel, dim3((unsigned)blocks), dim3(512), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ssd
