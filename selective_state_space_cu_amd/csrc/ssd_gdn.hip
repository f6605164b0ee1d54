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
//     O = scale (diag(gamma) Q H0 + (e^(G_i - G_j) q_i . k_j)_{j <= i} U)
//     H_next = gamma_last H0 + K^T diag(e^(G_last - G)) U
// (U_i is the delta-rule write value of token i; the token loop computes the
// same map one token at a time.)
//
// One workgroup per (sequence, value head, 64 value columns), four waves, one
// per SIMD: wave w owns value columns 16 w .. 16 w + 15 and carries their
// state rows S[v][0..dk) (float32, in the accumulator layout of the state
// update: register u, element r = S[16 w + q][16 u + 4 g + r] for lane
// (g, q)) from chunk to chunk. Per chunk, in order (barrier between phases):
//   load K, Q (64 x 128) and this slice of V (64 x 64) into LDS (zero rows past
//   the sequence: gate 0 and beta 0 make them neutral) and the gate / beta rows;
//   tables (cumsum, gamma, decay factors);
//   K K^T and Q K^T sub-tiles on the matrix cores, masked by the decay, into A
//   (float32) and the causal matrix Mq (bf16);
//   T: 16 x 16 diagonal blocks by forward substitution, then block rows below
//   (float32 VALU; exact to float32);
//   W^T = (beta gamma K)^T T^T, U^T = (beta V)^T T^T - H0^T W^T (bf16 matrix products,
//   float32 accumulation);
//   O^T = (H0^T Q^T) diag(gamma) + U^T Mq^T, scaled; the state update
//   H = gamma_last H + K^T (rho U), rho_j = e^(G_last - G_j); the state after
//   the chunk goes to its checkpoint slot when the plan names one.
#include <hip/hip_runtime.h>

#include "ssd_scan.hpp"

namespace ssd {

namespace {

constexpr int kGdnDk = 128;            // key dimension
constexpr int kGdnCols = 64;           // value columns per workgroup
constexpr int kGdnChunk = 64;          // tokens per chunk
// LDS layouts (bytes), those of the scan's general kernel: K rows in the B
// layout (pitch 288 + 128 per 8 rows: conflict-free row-fragment and
// transposed reads), Q and W rows in the C layout (pitch 272), V and U rows in
// the x layout (pitch 144), T and Mq rows in the decay-matrix layout (160).
constexpr int kPB = kGdnDk * 2 + 32, kGB = 8 * kPB + 128, kTileK = 8 * kGB;
constexpr int kPC = kGdnDk * 2 + 16, kTileQ = kGdnChunk * kPC;
constexpr int kPX = kGdnCols * 2 + 16, kTileV = kGdnChunk * kPX;
constexpr int kMPB = (kGdnChunk + 16) * 2, kTileM = kGdnChunk * kMPB;
constexpr int kPF = kGdnChunk + 1;     // float32 64 x 64 matrices: row pitch (floats)

__device__ __forceinline__ int gbrow(int r) { return (r >> 3) * kGB + (r & 7) * kPB; }

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ssd_gdn_chunk_kernel(GdnArgs a)
#if !defined(__HIP_DEVICE_COMPILE__)
{   // the host pass only needs the signature (for the launch stub)
}
#else
{
    using O = Ops<uint16_t>;
    using Frag = O::Frag;
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
    constexpr int DK = kGdnDk, CH = kGdnChunk;

    __shared__ __align__(16) unsigned char sK[kTileK];
    __shared__ __align__(16) unsigned char sQ[kTileQ];
    __shared__ __align__(16) unsigned char sV[kTileV];
    __shared__ __align__(16) unsigned char sW[kTileQ];
    __shared__ __align__(16) unsigned char sU[kTileV];
    __shared__ __align__(16) unsigned char sT[kTileM];
    __shared__ __align__(16) unsigned char sMq[kTileM];
    __shared__ __align__(16) float fA[CH * kPF];   // A (float32), then the state staging area (with fT)
    __shared__ __align__(16) float fT[CH * kPF];   // T (float32)
    // tables of the chunk: G (log2), gamma, beta, beta gamma, rho, V, Bf (64 each) and P (16)
    __shared__ __align__(16) float tab[7 * 64 + 16];
    float *const tG = tab, *const tGam = tab + 64, *const tBeta = tab + 128, *const tBG = tab + 192,
                 *const tRho = tab + 256, *const tVf = tab + 320, *const tBf = tab + 384, *const tP = tab + 448;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane & 15, g = lane >> 4;

    if (__builtin_nontemporal_load(a.error_flag) & SSD_DATA_BAD_CU_SEQLENS) return;
    const int b = blockIdx.x;
    const int per_seq = a.H * a.nptiles;
    const int rank = b / per_seq, rem = b - rank * per_seq;
    const int h = rem / a.nptiles, pt = rem - (rem / a.nptiles) * a.nptiles;
    const int s = a.seq_order[rank];
    if (s < 0 || s >= a.S) return;
    const int H = a.H, G = a.G, DV = a.dv;
    const int grp = h / (H / G);
    int64_t tb = a.cu_seqlens[s], te = a.cu_seqlens[s + 1];
    tb = tb < 0 ? 0 : (tb > a.T ? a.T : tb);
    te = te < tb ? tb : (te > a.T ? a.T : te);
    const int L = (int)(te - tb);
    const int nch = (L + CH - 1) / CH;
    const int c0 = a.seq_chunk_start[s];
    const int v0 = pt * kGdnCols;              // first value column of the workgroup
    const int vw = v0 + 16 * wave;             // first value column of this wave

    // state rows of this wave's 16 columns: st[u][r] = S[vw + q][16 u + 4 g + r]
    f32x4 st[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) st[u] = f32x4{0, 0, 0, 0};
    if (a.init != nullptr && (a.has_init == nullptr || a.has_init[s] != 0)) {
        const float *src = a.init + ((int64_t)(s * H + h) * DV + vw + q) * DK;
#pragma unroll
        for (int u = 0; u < 8; ++u) st[u] = *reinterpret_cast<const f32x4 *>(src + 16 * u + 4 * g);
    }

    // zero the strictly-upper sub-tiles that the causal products read
    // (row block 0 x column block 1, row block 2 x column block 3) in T and Mq
    {
        const int t2 = tid & 127, r = t2 >> 3, part = t2 & 7;   // 16 rows x 8 pieces of 4 bytes per sub-tile
        const int which = tid >> 7;                             // 0: sub-tile (0,1); 1: (2,3)
        const int I = which ? 2 : 0, row = 16 * I + r, col = 16 * (I + 1) + 2 * part;
        *reinterpret_cast<uint32_t *>(sT + row * kMPB + col * 2) = 0u;
        *reinterpret_cast<uint32_t *>(sMq + row * kMPB + col * 2) = 0u;
    }

    const float scale = a.scale;
    for (int c = 0; c < nch; ++c) {
        const int64_t t0 = tb + (int64_t)c * CH;
        const int Lc = min(CH, L - c * CH);

        // ---- load the chunk: K, Q rows (256 B), this slice of V (128 B), gate, beta
        {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int piece = tid + 256 * i, r = piece >> 4, cpos = piece & 15;   // 64 rows x 16 pieces
                u32x4 kv = {0, 0, 0, 0}, qv = {0, 0, 0, 0};
                if (r < Lc) {
                    const int64_t off = ((t0 + r) * G + grp) * DK + 8 * cpos;
                    kv = *reinterpret_cast<const u32x4 *>(a.k + off);
                    qv = *reinterpret_cast<const u32x4 *>(a.q + off);
                }
                *reinterpret_cast<u32x4 *>(sK + gbrow(r) + 16 * cpos) = kv;
                *reinterpret_cast<u32x4 *>(sQ + r * kPC + 16 * cpos) = qv;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int piece = tid + 256 * i, r = piece >> 3, cpos = piece & 7;    // 64 rows x 8 pieces
                u32x4 vv = {0, 0, 0, 0};
                if (r < Lc) vv = *reinterpret_cast<const u32x4 *>(a.v + ((t0 + r) * H + h) * DV + v0 + 8 * cpos);
                *reinterpret_cast<u32x4 *>(sV + r * kPX + 16 * cpos) = vv;
            }
            if (wave == 0) {   // tables from gate and beta (lane j = token j; 0 past the end)
                const float gt = lane < Lc ? a.gate[(t0 + lane) * H + h] * kLog2e : 0.0f;
                const float bt = lane < Lc ? a.beta[(t0 + lane) * H + h] : 0.0f;
                const float v = wave_scan(gt);   // inclusive cumsum (log2)
                const float e0 = readlane(v, 15), e1 = readlane(v, 31), e2 = readlane(v, 47), e3 = readlane(v, 63);
                const int blk = lane >> 4;
                const float s_prev = blk == 0 ? 0.0f : (blk == 1 ? e0 : (blk == 2 ? e1 : e2));
                const float s_end = blk == 0 ? e0 : (blk == 1 ? e1 : (blk == 2 ? e2 : e3));
                const float gam = fast_exp2(v);
                tG[lane] = v;
                tGam[lane] = gam;
                tBeta[lane] = bt;
                tBG[lane] = bt * gam;
                tRho[lane] = fast_exp2(e3 - v);
                tVf[lane] = fast_exp2(v - s_prev);     // e^(G_i - G_end(block(i) - 1))
                tBf[lane] = fast_exp2(s_end - v);      // e^(G_end(block(j)) - G_j)
                if (lane < 16) {
                    const int J = lane >> 2, dd = lane & 3, I = J + dd;
                    const float ea = I == 1 ? e0 : (I == 2 ? e1 : e2), eb = J == 0 ? e0 : (J == 1 ? e1 : e2);
                    tP[lane] = dd == 0 ? 1.0f : (I >= 4 ? 0.0f : fast_exp2(ea - eb));   // e^(G_end(I-1) - G_end(J))
                }
            }
        }
        lds_barrier();

        // ---- K K^T and Q K^T sub-tiles (I, J = w), I = w .. 3, masked by the decay:
        //      A[i][j] = beta_i e^(G_i - G_j) k_i.k_j (j < i, float32), Mq[i][j] = e^(G_i - G_j) q_i.k_j (j <= i, bf16)
        {
            const int J = wave;
            Frag kj[4];   // K rows of column block J (row fragments, permuted k order)
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) kj[kc] = O::rowk_perm(sK + gbrow(16 * J + q) + (32 * kc + 4 * g) * 2);
            float sj[4], bfj[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sj[r] = tG[16 * J + 4 * g + r];
                bfj[r] = tBf[16 * J + 4 * g + r];
            }
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (I < J) continue;
                f32x4 kk = {0, 0, 0, 0}, qk = {0, 0, 0, 0};
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    kk = O::mma(kk, kj[kc], O::rowk_perm(sK + gbrow(16 * I + q) + (32 * kc + 4 * g) * 2));
                    qk = O::mma(qk, kj[kc], O::rowk_perm(sQ + (16 * I + q) * kPC + (32 * kc + 4 * g) * 2));
                }
                // lane (g, q): i = 16 I + q, j = 16 J + 4 g + r
                const int i = 16 * I + q;
                const float bi = tBeta[i];
                float fa[4], fq[4];
                if (I == J) {
                    const float si = tG[i];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int jr = 4 * g + r;
                        const float f = jr <= q ? fast_exp2(si - sj[r]) : 0.0f;
                        fq[r] = qk[r] * f;
                        fa[r] = jr < q ? bi * kk[r] * f : 0.0f;
                    }
                } else {
                    const float rowf = tVf[i] * tP[4 * J + (I - J)];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float f = rowf * bfj[r];
                        fq[r] = qk[r] * f;
                        fa[r] = bi * kk[r] * f;
                    }
                }
                float *ar = fA + i * kPF + 16 * J + 4 * g;
#pragma unroll
                for (int r = 0; r < 4; ++r) ar[r] = fa[r];
                O::mstore4(sMq + i * kMPB + (16 * J + 4 * g) * 2, fq);
            }
        }
        lds_barrier();

        // ---- T = (I + A)^-1: diagonal blocks by forward substitution (wave w: block w,
        //      lane j < 16 owns column j): T[i][j] = [i == j] - sum_{j <= m < i} A[i][m] T[m][j]
        {
            const int base = 16 * wave;
            if (lane < 16) {
                float tc[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float acc = i == lane ? 1.0f : 0.0f;
#pragma unroll
                    for (int m = 0; m < i; ++m) acc -= fA[(base + i) * kPF + base + m] * tc[m];
                    tc[i] = i < lane ? 0.0f : acc;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) fT[(base + i) * kPF + base + lane] = tc[i];
            }
        }
        lds_barrier();
        // blocks below the diagonal, by distance from it (wave w: block (w + dist, w)):
        //   T_IJ = -T_II X,  X = sum_{J <= K < I} A_IK T_KJ   (16 x 16 float32 products on the
        //   VALU; lane: row lane / 4, columns 4 (lane mod 4) ..), X staged through the unused
        //   strictly-upper part of A (row block J, column block I)
#pragma unroll
        for (int dist = 1; dist < 4; ++dist) {
            if (wave + dist < 4) {
                const int J = wave, I = wave + dist;
                const int r = lane >> 2, c4 = 4 * (lane & 3);
                float x[4] = {0, 0, 0, 0};
                for (int K = J; K < I; ++K)
                    for (int m = 0; m < 16; ++m) {
                        const float aim = fA[(16 * I + r) * kPF + 16 * K + m];
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = fmaf(aim, fT[(16 * K + m) * kPF + 16 * J + c4 + e], x[e]);
                    }
                float *xs = fA + (16 * J + r) * kPF + 16 * I + c4;   // row block J, column block I: unused by A
#pragma unroll
                for (int e = 0; e < 4; ++e) xs[e] = x[e];
                __builtin_amdgcn_wave_barrier();
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                float t4[4] = {0, 0, 0, 0};
                for (int m = 0; m < 16; ++m) {
                    const float tim = fT[(16 * I + r) * kPF + 16 * I + m];
#pragma unroll
                    for (int e = 0; e < 4; ++e) t4[e] = fmaf(tim, fA[(16 * J + m) * kPF + 16 * I + c4 + e], t4[e]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) fT[(16 * I + r) * kPF + 16 * J + c4 + e] = -t4[e];
            }
            lds_barrier();
        }
        // T (lower, unit diagonal) -> bf16 tile: the 10 lower sub-tiles
        for (int idx = tid; idx < 10 * 64; idx += 256) {
            static constexpr int kI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3}, kJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
            const int sub = idx >> 6, e = idx & 63, r = e >> 2, c4 = 4 * (e & 3);
            const int I = kI[sub], J = kJ[sub], i = 16 * I + r;
            float v4[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int j = 16 * J + c4 + x;
                v4[x] = j <= i ? fT[i * kPF + j] : 0.0f;
            }
            O::mstore4(sT + i * kMPB + (16 * J + c4) * 2, v4);
        }
        lds_barrier();

        // ---- W^T = (beta gamma K)^T T^T: wave w computes key rows 32 w .. 32 w + 31 (u = 2 w, 2 w + 1)
        {
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
                const int u = 2 * wave + uu;
                Frag kt[2];   // (beta gamma K)^T fragments: key column 16 u + q, tokens 32 ks + 8 g + slot
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const Frag raw = O::tr(sK + gbrow(32 * ks + 8 * g) + O::tr_row(q) * kPB + (16 * u + O::tr_col(q)) * 2,
                                           4 * kPB);
                    float w8[8];
#pragma unroll
                    for (int sl = 0; sl < 8; ++sl) w8[sl] = tBG[32 * ks + 8 * g + sl];
                    kt[ks] = O::scale(raw, w8);
                }
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        if (ks <= d / 2) acc = O::mma(acc, kt[ks], O::mrow(sT + (16 * d + q) * kMPB + (32 * ks + 8 * g) * 2));
                    // acc[r] = W[token 16 d + q][key 16 u + 4 g + r]
                    const float w4[4] = {acc[0], acc[1], acc[2], acc[3]};
                    O::mstore4(sW + (16 * d + q) * kPC + (16 * u + 4 * g) * 2, w4);
                }
            }
        }
        lds_barrier();

        // ---- U^T = (beta V)^T T^T - H0^T W^T (this wave's 16 value columns) -> U tile
        Frag hf[4];   // H0^T = S0 rows as operands: k step c covers keys 32 c .. + 31 (permuted order)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) hf[kc] = O::from_f32(st[2 * kc], st[2 * kc + 1]);
        {
            Frag vf[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const Frag raw = O::tr(sV + (32 * ks + 8 * g + O::tr_row(q)) * kPX + (16 * wave + O::tr_col(q)) * 2, 4 * kPX);
                float w8[8];
#pragma unroll
                for (int sl = 0; sl < 8; ++sl) w8[sl] = tBeta[32 * ks + 8 * g + sl];
                vf[ks] = O::scale(raw, w8);
            }
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                f32x4 u1 = {0, 0, 0, 0}, u2 = {0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks <= d / 2) u1 = O::mma(u1, vf[ks], O::mrow(sT + (16 * d + q) * kMPB + (32 * ks + 8 * g) * 2));
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    u2 = O::mma(u2, hf[kc], O::rowk_perm(sW + (16 * d + q) * kPC + (32 * kc + 4 * g) * 2));
                // (u1 - u2)[r] = U[token 16 d + q][value column 16 w + 4 g + r]
                const float uv[4] = {u1[0] - u2[0], u1[1] - u2[1], u1[2] - u2[2], u1[3] - u2[3]};
                *(uint2 *)(sU + (16 * d + q) * kPX + (16 * wave + 4 * g) * 2) =
                    uint2{pack_bf16(uv[0], uv[1]), pack_bf16(uv[2], uv[3])};
            }
        }
        lds_barrier();

        // ---- O^T = scale ((H0^T Q^T) diag(gamma) + U^T Mq^T); then the state update
        //      H = gamma_last H + K^T (rho o U)
        {
            Frag uf[2];   // U^T fragments: value column 16 w + q, tokens 32 ks + 8 g + slot
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                uf[ks] = O::tr(sU + (32 * ks + 8 * g + O::tr_row(q)) * kPX + (16 * wave + O::tr_col(q)) * 2, 4 * kPX);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                f32x4 o1 = {0, 0, 0, 0}, o2 = {0, 0, 0, 0};
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    o1 = O::mma(o1, hf[kc], O::rowk_perm(sQ + (16 * d + q) * kPC + (32 * kc + 4 * g) * 2));
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks <= d / 2) o2 = O::mma(o2, uf[ks], O::mrow(sMq + (16 * d + q) * kMPB + (32 * ks + 8 * g) * 2));
                const int i = 16 * d + q;
                const float gi = tGam[i];
                if (i < Lc) {
                    uint16_t *dst = a.o + ((t0 + i) * H + h) * DV + vw + 4 * g;
                    *(uint2 *)dst = uint2{pack_bf16(scale * fmaf(o1[0], gi, o2[0]), scale * fmaf(o1[1], gi, o2[1])),
                                          pack_bf16(scale * fmaf(o1[2], gi, o2[2]), scale * fmaf(o1[3], gi, o2[3]))};
                }
            }
            // state update: st[u] (key rows 16 u + 4 g + r, value column q) = gamma_last st[u] + sum_ks Kt[u] (rho U)
            Frag ru[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float w8[8];
#pragma unroll
                for (int sl = 0; sl < 8; ++sl) w8[sl] = tRho[32 * ks + 8 * g + sl];
                ru[ks] = O::scale(uf[ks], w8);
            }
            const float gl = tGam[63];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                st[u] *= gl;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    st[u] = O::mma(st[u],
                                   O::tr(sK + gbrow(32 * ks + 8 * g) + O::tr_row(q) * kPB + (16 * u + O::tr_col(q)) * 2, 4 * kPB),
                                   ru[ks]);
            }
        }
        // the state after the chunk into its checkpoint slot
        if (a.chunk_states != nullptr) {
            const int gc = c0 + c;
            int dsl = (gc >= 0 && gc < a.max_chunks) ? (a.chunk_state_dst ? a.chunk_state_dst[gc] : gc) : -1;
            if (dsl >= a.capacity) {
                if (tid == 0) atomicOr(a.error_flag, SSD_DATA_BAD_SLOT);
                dsl = -1;
            }
            if (dsl >= 0) {
                float *dst = a.chunk_states + ((int64_t)dsl * H + h) * DV * DK + (int64_t)(vw + q) * DK;
#pragma unroll
                for (int u = 0; u < 8; ++u) *reinterpret_cast<f32x4 *>(dst + 16 * u + 4 * g) = st[u];
            }
        }
        lds_barrier();   // the chunk's tiles are consumed before the next chunk's loads
    }

    float *fd = a.final_states + ((int64_t)(s * H + h) * DV + vw + q) * DK;
#pragma unroll
    for (int u = 0; u < 8; ++u) *reinterpret_cast<f32x4 *>(fd + 16 * u + 4 * g) = st[u];
}
#endif

hipError_t launch_gdn(const GdnArgs &a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.S * a.H * a.nptiles;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(ssd_gdn_chunk_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ssd
