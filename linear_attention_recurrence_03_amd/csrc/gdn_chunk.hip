// gdn_chunk.hip -- chunked form of the gated delta rule for gfx950.
//
// The token recurrence (state M stored [value][key]; per token
// M <- e^g M, delta = beta (v - M k), M <- M + delta k^T, out = M q / sqrt(d))
// is rewritten over chunks of C = 64 tokens so that the work inside a chunk is
// dense matrix products ("Gated Delta Net on AMD", velstech.net, section "Why
// this bites AMD users specifically": the fused chunked kernel reformulates the
// recurrence to run in parallel blocks).  For one chunk starting from state
// M_n, with gam_r the inclusive sum of g over the chunk's first r+1 tokens:
//
//   A[r][s] = beta_r e^{gam_r - gam_s} (k_r . k_s)   s < r     (strictly lower)
//   T       = (I + A)^{-1}                                    (unit lower)
//   E       = diag(beta) (V - diag(e^gam) K M_n^T)             state dependent
//   Delta   = T E                      row r = the delta vector of token r
//   P[r][s] = e^{gam_r - gam_s} (q_r . k_s)           s <= r
//   O       = (diag(e^gam) Q M_n^T + P Delta) / sqrt(d)
//   M_{n+1} = e^{gam_last} M_n + (diag(e^{gam_last - gam}) Delta)^T K
//
// Only differences gam_r - gam_s with s <= r are exponentiated, so strong decay
// underflows to zero instead of overflowing.
//
// Two kernels run per call, the prep and one of three chunk-to-chunk passes:
//   chunk_prep_kernel  -- one workgroup per (seq, head, chunk), all chunks in
//                         parallel: the state-independent part (gates, A, T, P).
//                         K K^T and Q K^T run on MFMA; T comes from a blocked
//                         triangular inverse in LDS (16x16 diagonal blocks by
//                         forward substitution, then the off-diagonal blocks).
//                         Writes T, the gate vectors and (unless the pass forms
//                         it itself) P to the workspace.
//   chunk_scan_kernel  -- one workgroup per (seq, head, block of value rows),
//                         walking the chunks in order and carrying its rows of
//                         M in registers.  Value rows of M are independent given
//                         k, q, g, beta, so splitting them across workgroups
//                         needs no communication.  Each 16-row value tile has
//                         three waves on MFMA (16x16x32 bf16 for bf16 inputs,
//                         16x16x4 fp32 for fp32 inputs): X forms K M^T, E and
//                         T E, U holds the tile's rows of M and updates them, O
//                         forms Q M^T and P Delta.  Four producer waves move the
//                         chunk's K, Q, T, P, V and gates into LDS by LDS-DMA
//                         (K^T operands come from transposing LDS reads), the
//                         next chunks' loads in flight while one is computed.
//   chunk_head_kernel  -- (bf16, from one (seq, head) per compute unit on) one
//                         workgroup per (seq, head) carrying all its value rows
//                         (gdn_chunk_head.hip).
//   chunk_lag_kernel   -- (bf16, on request) the two-chunk-lag form of the pass
//                         (gdn_chunk_lag.hip).
// This file holds the prep, the per-tile pass and the choice between the passes;
// the MFMA fragment conventions and helpers they share are in gdn_chunk_common.h.
#include "gdn_chunk_common.h"

namespace gdn {
namespace {

// The products of one prep wave: the lower tiles of row tiles R0 and R1 of
// K K^T (KK) or Q K^T, kept in registers across the barrier that frees the K
// rows.  K rows come from LDS; Q rows from `fq` (row tile R0's D / 32 operand
// fragments, then R1's).  Each tile is formed transposed (K rows as the MFMA's A operand), so that
// lane (g, i) holds entries (16 tr + i, 16 tc + 4g + j), j = 0..3: four
// consecutive columns of one row.  K K^T tiles are already
// A = beta_r e^{gam_r - gam_s} (k_r . k_s) for s < r; Q K^T tiles are
// P = e^{gam_r - gam_s} (q_r . k_s) / sqrt(d) for s <= r.  A diagonal tile of K K^T is
// symmetric before the scaling, so it also gives the lane the diagonal block's
// entries (16 tr + 4g + j, 16 tr + i): those go, as the transposed fp32 block
// the forward substitution reads, to sD.  Tile (i, tc) is acc[i ? R0 + 1 + tc : tc].
template <int R0, int R1>
struct PrepTiles {
    static constexpr int N = R0 + 1 + R1 + 1;
    floatx4 acc[N];
};

template <int D, bool BF16, bool KK, int R0, int R1>
__device__ __forceinline__ void prep_products(PrepTiles<R0, R1> &pt, const unsigned char *smem,
                                              const float *sG, float *sD, const float *sN,
                                              int lane, const Frag<BF16> *fq)
{
    static_assert(R0 < R1, "row tiles");
    using L = PrepSmem<D, BF16>;
    constexpr int KS = D / 32;
    const int gq = lane >> 4, cl = lane & 15;
    const unsigned char *sK = smem + L::kK;
    // operands of the two row tiles: K rows (K K^T) or the Q rows already in registers
    Frag<BF16> fa[2][KS];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (KK) fa[i][ks] = row_frag<BF16>(sK, L::RK, 16 * (i ? R1 : R0) + cl, 32 * ks, gq);
            else fa[i][ks] = fq[i * KS + ks];
        }
    // column tiles in order, each column tile's K rows read once for both row tiles
    // (for K K^T the row tiles' own operands serve as their column tiles)
#pragma unroll
    for (int tc = 0; tc <= R1; ++tc) {
        Frag<BF16> kc[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (KK && tc == R0) kc[ks] = fa[0][ks];
            else if (KK && tc == R1) kc[ks] = fa[1][ks];
            else kc[ks] = row_frag<BF16>(sK, L::RK, 16 * tc + cl, 32 * ks, gq);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tr = i ? R1 : R0;
            if (tc > tr) continue;
            const int row = 16 * tr + cl;
            const float g_row = sG[row];
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mma(kc[ks], fa[i][ks], acc);
            const int col0 = 16 * tc + 4 * gq;
            if (sN) {  // normalised rows: (x_r / |x_r|) . (k_s / |k_s|)
                const float rr = sN[(KK ? 0 : C) + row];
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] *= rr * sN[col0 + j];
            }
            if (KK && tc == tr) {
                // sD[tr][m][r] = A[16 tr + r][16 tr + m]: entry (col0 + j, row) of the
                // symmetric tile, scaled as row col0 + j of A
                float d[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r2 = col0 + j;
                    const float e2 = __expf(sG[r2] - g_row);
                    d[j] = (row < r2) ? sG[C + r2] * e2 * acc[j] : 0.f;
                }
                *reinterpret_cast<float4 *>(sD + (tr * 16 + cl) * L::LDD + 4 * gq) =
                    make_float4(d[0], d[1], d[2], d[3]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = col0 + j;
                const float e = __expf(g_row - sG[col]);
                acc[j] = KK ? ((col < row) ? sG[C + row] * e * acc[j] : 0.f)
                            : ((col <= row) ? kOutScale<D> * e * acc[j] : 0.f);
            }
            pt.acc[i ? R0 + 1 + tc : tc] = acc;
        }
    }
}

// Writes a wave's A tiles into a C x C matrix of E (row stride ld elements): four
// consecutive columns of one row per lane and tile.
template <bool BF16, int R0, int R1>
__device__ __forceinline__ void store_tiles(const PrepTiles<R0, R1> &pt, typename Elem<BF16>::T *m,
                                            int ld, int lane)
{
    const int gq = lane >> 4, cl = lane & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tr = i ? R1 : R0;
#pragma unroll
        for (int tc = 0; tc <= (i ? R1 : R0); ++tc) {
            const floatx4 &a = pt.acc[i ? R0 + 1 + tc : tc];
            typename Elem<BF16>::T *dst = m + (16 * tr + cl) * ld + 16 * tc + 4 * gq;
            if constexpr (BF16)
                *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2(a[0], a[1]), pack2(a[2], a[3]));
            else
                *reinterpret_cast<float4 *>(dst) = make_float4(a[0], a[1], a[2], a[3]);
        }
    }
}

// P straight to the workspace: the fragment unit of block (row tile tt, k half h)
// that lane (g, i) owns holds row 16 tt + i, columns 32 h + 4g + j and
// 32 h + 16 + 4g + j, i.e. tiles (tt, 2h) and (tt, 2h + 1) of this lane (zero
// above the diagonal).  The wave owns every block of its two row tiles.
template <bool BF16, int R0, int R1>
__device__ __forceinline__ void emit_p(const PrepTiles<R0, R1> &pt, unsigned char *wp, int lane)
{
    constexpr int FB = kFragBytes<BF16>;
    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    unsigned char *unit = wp + FB * blk_unit(lane & 15, lane >> 4);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tt = i ? R1 : R0;
        const int base = i ? R0 + 1 : 0;
#pragma unroll
        for (int h = 0; 32 * h <= 16 * tt + 15; ++h) {
            const int b = tt < 2 ? tt : 2 * tt - 2 + h;
            const floatx4 &c0 = pt.acc[base + 2 * h];
            const int i1 = base + 2 * h + 1 < PrepTiles<R0, R1>::N ? base + 2 * h + 1 : 0;
            const floatx4 &c1 = (2 * h + 1 <= tt) ? pt.acc[i1] : zero4;
            const Frag<BF16> f = acc_frag<BF16>(c0, c1);
            uint4 w[FB / 16];
            __builtin_memcpy(w, &f, FB);
#pragma unroll
            for (int x = 0; x < FB / 16; ++x)
                reinterpret_cast<uint4 *>(unit + b * kBlkBytes<BF16>)[x] = w[x];
        }
    }
}

// Prep timestamps (trace builds only): wave 0 of each of the first kPrepTraceGroups
// workgroups records the shader clock at the start, when the chunk's rows have
// landed, after the products, after the diagonal inverses, after the two levels of
// off-diagonal blocks and at the end; gdn_prep_trace_read copies them out.
#ifdef GDN_PHASE_TRACE
constexpr int kPrepTraceGroups = 4096;
__device__ uint64_t g_prep_trace[kPrepTraceGroups][8];
#endif

struct PrepTrace {
    __device__ __forceinline__ void mark(int slot, int wave, int lane) const
    {
#ifdef GDN_PHASE_TRACE
        if (blockIdx.x < kPrepTraceGroups && wave == 0 && lane == 0)
            g_prep_trace[blockIdx.x][slot] = __builtin_amdgcn_s_memtime();
#else
        (void)slot;
        (void)wave;
        (void)lane;
#endif
    }
};

// One workgroup per (seq, head, chunk): the state-independent part of the chunk.
//   0. K rows -> LDS by LDS-DMA (all waves); Q rows -> operand registers
//      (waves 2, 3); gate sums (wave 0)
//   1. K K^T (waves 0, 1) and Q K^T (waves 2, 3) on MFMA, row tiles {0, 3} and
//      {1, 2} per wave so that each does five tiles; results stay in registers,
//      and waves 2, 3 write P to the workspace from them
//   2. the K space is reused: waves 0, 1 store A; wave 0 then inverts the
//      diagonal 16x16 blocks of I + A by forward substitution (lane = (block,
//      column), right-looking over a transposed fp32 copy of the block); wave 1
//      zeroes the blocks of T read before they are formed
//   3. blocks (1,0), (3,2): T_ij = -T_ii (A_ij T_jj)                (waves 0, 1)
//   4. blocks (2,0), (2,1), (3,0), (3,1): with the 32-row halves,
//      T_hi,lo = -T_hi (A_hi,lo T_lo)                              (waves 0, 1)
//   5. T to the workspace as six fragment blocks
// The products of steps 3 and 4 run on MFMA with the k range padded to 32 by
// blocks of T that are still zero; for bf16 inputs their operands are bf16.
// Register budget of the prep kernel, as workgroups per CU: what the LDS allows,
// except that fp32 rows of 128 with normalisation need more than 128 registers.
// The lag form's prep (bf16) also holds the key rows of the two previous chunks
// and the scaled cross products, and runs three per CU (four spill registers; with
// normalised rows at d=128 two, as three spill).
template <int D, bool BF16, bool NORM, bool LAG>
constexpr int prep_per_cu()
{
    return LAG ? ((NORM && D >= 128) ? 2 : PrepSmem<D, BF16>::kPerCU > 3 ? 3 : PrepSmem<D, BF16>::kPerCU)
         : (!BF16 && NORM && D >= 128 && PrepSmem<D, BF16>::kPerCU > 3) ? 3
                                                                       : PrepSmem<D, BF16>::kPerCU;
}

// Sum of squares of the elements in 16 bytes (eight bf16 or four fp32), added to acc.
template <bool BF16>
__device__ __forceinline__ float sumsq16(const uint4 &u, float acc)
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (BF16) {
            const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xffff0000u);
            acc = fmaf(lo, lo, fmaf(hi, hi, acc));
        } else {
            const float f = __uint_as_float(w[e]);
            acc = fmaf(f, f, acc);
        }
    }
    return acc;
}

// LAG (bf16 only): also R1 and R2, the lag form's cross-chunk matrices, and the
// WsLag workspace layout.  Each wave w forms column tile w of K_n K_{n-1}^T and
// K_n K_{n-2}^T from the K rows in LDS and the earlier chunks' rows 16w..16w+15
// held as B operands, scales row s by -beta_s e^{gam_s} (and e^{c_{n-1}} for R2),
// keeps the result as two bf16 A operands (k = the rows s of chunk n), and once T
// is final multiplies by T: (T Y)^T = Y^T T^T, whose accumulator hands lane (g, i)
// four consecutive columns of row i, i.e. half of a fragment unit.
template <int D, bool BF16, bool NORM, bool LAG, bool PQ>
__global__ __launch_bounds__(kPrepThreads)
__attribute__((amdgpu_waves_per_eu(prep_per_cu<D, BF16, NORM, LAG>()))) void chunk_prep_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, unsigned char *__restrict__ ws, int64_t n_tokens,
    int64_t n_heads, int64_t n_k_heads, int n_chunks, int raw_gates)
{
    static_assert(!LAG || BF16, "the lag form runs on bf16 rows");
    using E = typename Elem<BF16>::T;
    using L = PrepSmem<D, BF16>;
    using W = WsLayout<BF16>;
    static_assert(PQ || (BF16 && !NORM && !LAG), "P is left to the pass only for plain bf16 rows");
    // without P (the whole-head pass forms it) the gates take the 2 KiB area, with a
    // sixth row holding gam itself
    constexpr int64_t kStride = LAG ? WsLag::kBytes : !PQ ? W::kBytesNorm : W::stride(NORM);
    constexpr int64_t kWsP = LAG ? WsLag::kP : W::kP;
    constexpr int64_t kWsT = LAG ? WsLag::kT : W::kT;
    constexpr int64_t kWsG = LAG ? WsLag::kGates : W::kGates;
    constexpr int LDT = L::LDT;
    extern __shared__ __align__(16) unsigned char smem[];
    E *sT = reinterpret_cast<E *>(smem + L::kT);
    E *sAe = reinterpret_cast<E *>(smem + L::kAe);
    float *sD = reinterpret_cast<float *>(smem + L::kD);
    float *sG = reinterpret_cast<float *>(smem + L::kG);  // gam, beta, e^gam, e^{last-gam}, e^last

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gq = lane >> 4, cl = lane & 15;
    // Blocks are numbered chunk-major (every (seq, head) of chunk n, then chunk n+1;
    // the grid is exactly n_sh * n_chunks): all heads of a token are contiguous in q
    // and k, so each round of workgroups reads whole token rows.  The workspace stays
    // (seq, head)-major.
    const int64_t n_sh = gridDim.x / n_chunks;
    const int n = static_cast<int>(blockIdx.x / n_sh);
    const int64_t sh = blockIdx.x - int64_t(n) * n_sh;
    const int64_t chunk_id = sh * n_chunks + n;
    const int64_t s = sh / n_heads, h = sh - s * n_heads;
    const int64_t t0 = int64_t(n) * C;
    const int nv = static_cast<int>(min<int64_t>(C, n_tokens - t0));
    unsigned char *dst = ws + chunk_id * kStride;
    const PrepTrace ptr;
    ptr.mark(0, wave, lane);

    // 0. K rows of key head h % n_k_heads into LDS; waves 2 and 3 load the Q rows
    //    of their row tiles ({0, 3} and {1, 2}) as MFMA operands (lane (g, i): row
    //    16 tr + i, k = 8g .. 8g + 7 of each 32-wide k step).  Rows past the end
    //    repeat the last valid one: their A and P entries are cleared by beta = 0
    //    and never read.  Then the gates.
    constexpr int KS = D / 32;
    Frag<BF16> fq[2 * KS];
    {
        const int64_t off = ((s * n_tokens + t0) * n_k_heads + h % n_k_heads) * D * L::ES;
        const unsigned char *kb = static_cast<const unsigned char *>(k) + off;
        const unsigned char *qb = static_cast<const unsigned char *>(q) + off;
        const uint32_t hdb = static_cast<uint32_t>(n_k_heads * D * L::ES);
        for (int i = wave; i < L::NBK; i += kPrepThreads / 64)
            dma16(kb, dma_src_offset(i, lane, D * L::ES, L::RK, hdb, nv), smem + L::kK + 1024 * i);
        if (PQ && wave >= 2) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tr = (wave == 2) ? (i ? 3 : 0) : (i ? 2 : 1);
                const unsigned char *src =
                    qb + int64_t(min(16 * tr + cl, nv - 1)) * hdb + 8 * gq * L::ES;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    fq[i * KS + ks] = *reinterpret_cast<const Frag<BF16> *>(src + 32 * ks * L::ES);
            }
        }
    }
    // LAG: rows 16 w .. 16 w + 15 of chunks n-1 and n-2 as B operands (lane (g, i):
    // row 16 w + i, k = 8g .. 8g + 7 of each 32-wide step); zero rows for chunks
    // before the first, which makes R1 and R2 zero there
    Frag<BF16> kp1[LAG ? KS : 1], kp2[LAG ? KS : 1];
    if constexpr (LAG) {
        const int64_t hk = h % n_k_heads;
        const int64_t hdb = n_k_heads * D * L::ES;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kp1[ks].u = make_uint4(0u, 0u, 0u, 0u);
            kp2[ks].u = make_uint4(0u, 0u, 0u, 0u);
        }
        if (n >= 1) {
            const unsigned char *src = static_cast<const unsigned char *>(k) +
                ((s * n_tokens + t0 - C + 16 * wave + cl) * n_k_heads + hk) * D * L::ES +
                8 * gq * L::ES;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kp1[ks] = *reinterpret_cast<const Frag<BF16> *>(src + 32 * ks * L::ES);
            if (n >= 2) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kp2[ks] = *reinterpret_cast<const Frag<BF16> *>(src - C * hdb + 32 * ks * L::ES);
            }
        }
    }
    if (wave == 0) {
        float gv = 0.f, bv = 0.f;
        if (lane < nv) {
            const int64_t gi = (s * n_tokens + t0 + lane) * n_heads + h;
            gv = g[gi];
            bv = beta[gi];
            if (raw_gates) {
                gv = neg_softplus(gv);
                bv = sigmoid(bv);
            }
        }
        float x = gv;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        const float glast = __shfl(x, nv - 1, 64);
        const bool ok = lane < nv;
        sG[lane] = x;
        sG[C + lane] = ok ? bv : 0.f;
        sG[2 * C + lane] = ok ? expf(x) : 0.f;
        sG[3 * C + lane] = ok ? expf(glast - x) : 0.f;
        if (lane == 0) sG[4 * C] = expf(glast);
    } else if (LAG && wave == 1) {
        // e^{c_{n-1}}: the decay of the whole previous chunk (used by R2 only)
        float gp = 0.f;
        if (n >= 1) {
            gp = g[(s * n_tokens + t0 - C + lane) * n_heads + h];
            if (raw_gates) gp = neg_softplus(gp);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) gp += __shfl_xor(gp, o, 64);
        if (lane == 0) sG[4 * C + 1] = expf(gp);
    }
    wait_vmem_le<0>();
    lds_barrier();
    ptr.mark(1, wave, lane);

    // 0b. normalised rows: 1 / sqrt(|x_r|^2 + eps) for the K rows (waves 0, 1: 32
    //     rows each, two lanes per row, from LDS) and the Q rows (waves 2, 3: their
    //     row tiles, from the operand registers, four lanes per row)
    float *sN = nullptr;
    if constexpr (NORM) {
        sN = reinterpret_cast<float *>(smem + L::kN);
        if (wave < 2) {
            const int r = 32 * wave + (lane & 31), half = lane >> 5;
            constexpr int HB = D * L::ES / 2;  // bytes of half a row
            const unsigned char *row = smem + L::kK + r * L::RK + half * HB;
            float acc = 0.f;
#pragma unroll
            for (int o = 0; o < HB; o += 16) acc = sumsq16<BF16>(*reinterpret_cast<const uint4 *>(row + o), acc);
            acc += __shfl_xor(acc, 32, 64);
            if (half == 0) sN[r] = 1.f / sqrtf(acc + kL2Eps);
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tr = (wave == 2) ? (i ? 3 : 0) : (i ? 2 : 1);
                float acc = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    uint4 w[sizeof(Frag<BF16>) / 16];
                    __builtin_memcpy(w, &fq[i * KS + ks], sizeof(w));
#pragma unroll
                    for (int x = 0; x < int(sizeof(w) / 16); ++x) acc = sumsq16<BF16>(w[x], acc);
                }
                acc += __shfl_xor(acc, 16, 64);
                acc += __shfl_xor(acc, 32, 64);
                if (gq == 0) sN[C + 16 * tr + cl] = 1.f / sqrtf(acc + kL2Eps);
            }
        }
        lds_barrier();
    }

    // LAG: Y1 = -diag(beta e^gam) K_n K_{n-1}^T and Y2 = e^{c_{n-1}} Y1's form with
    // K_{n-2}, column tile w, as bf16 A operands of their transposes (k = rows of
    // chunk n in fragment order, two 32-row halves)
    Frag<BF16> y1[2], y2[2];
    if constexpr (LAG) {
        const unsigned char *sK = smem + L::kK;
        // one matrix at a time: its four accumulator tiles, then two bf16 operands
        auto cross = [&](const Frag<BF16> (&kp)[KS], float scale, Frag<BF16> (&y)[2]) {
            floatx4 x[4];
#pragma unroll
            for (int ts = 0; ts < 4; ++ts) {
                x[ts] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    x[ts] = mma(row_frag<BF16>(sK, L::RK, 16 * ts + cl, 32 * ks, gq), kp[ks], x[ts]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r = 16 * ts + 4 * gq + jj;
                    float f = -scale * sG[C + r] * sG[2 * C + r];
                    if constexpr (NORM) f *= sN[r];
                    x[ts][jj] *= f;
                }
            }
            y[0] = acc_frag<BF16>(x[0], x[1]);
            y[1] = acc_frag<BF16>(x[2], x[3]);
        };
        cross(kp1, 1.f, y1);
        cross(kp2, sG[4 * C + 1], y2);
    }

    // 1-2. products, then the reuse of the K space
    if (wave < 2) {
        if (wave == 0) {
            PrepTiles<0, 3> pt;
            prep_products<D, BF16, true, 0, 3>(pt, smem, sG, sD, sN, lane, nullptr);
            lds_barrier();
            store_tiles<BF16, 0, 3>(pt, sAe, LDT, lane);
            ptr.mark(2, wave, lane);
        } else {
            PrepTiles<1, 2> pt;
            prep_products<D, BF16, true, 1, 2>(pt, smem, sG, sD, sN, lane, nullptr);
            lds_barrier();
            store_tiles<BF16, 1, 2>(pt, sAe, LDT, lane);
        }
    } else {
        if (wave == 2) {
            if constexpr (PQ) {
                PrepTiles<0, 3> pt;
                prep_products<D, BF16, false, 0, 3>(pt, smem, sG, sD, sN, lane, fq);
                emit_p<BF16, 0, 3>(pt, dst + kWsP, lane);
            }
            lds_barrier();
        } else {
            if constexpr (PQ) {
                PrepTiles<1, 2> pt;
                prep_products<D, BF16, false, 1, 2>(pt, smem, sG, sD, sN, lane, fq);
                emit_p<BF16, 1, 2>(pt, dst + kWsP, lane);
            }
            lds_barrier();
            // beta, e^gam, e^{last-gam}, e^last; with normalised rows the second and
            // third carry 1/|k| and a fifth row holds e^gam / |q|
            float *wG = reinterpret_cast<float *>(dst + kWsG);
            const float rk = sN ? sN[lane] : 1.f;
            wG[lane] = sG[C + lane];
            wG[C + lane] = sG[2 * C + lane] * rk;
            wG[2 * C + lane] = sG[3 * C + lane] * rk;
            wG[3 * C + lane] = sG[4 * C];
            if (LAG || sN) wG[4 * C + lane] = sG[2 * C + lane] * (sN ? sN[C + lane] : 1.f);
            if (!PQ) wG[5 * C + lane] = sG[lane];
        }
    }
    if (wave == 0) {
        // diagonal blocks of T = (I + A)^{-1}: lane = (block b, column c); after
        // x[m] is final it is eliminated from the rows below it
        const int b = lane >> 4, c = lane & 15;
        const float *Ab = sD + b * 16 * L::LDD;  // Ab[m * LDD + r] = A[16b + r][16b + m]
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
        float4 cur[4], nxt[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) cur[v] = *reinterpret_cast<const float4 *>(Ab + 4 * v);
#pragma unroll
        for (int m = 0; m < 15; ++m) {
            if (m + 1 < 15) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    nxt[v] = *reinterpret_cast<const float4 *>(Ab + (m + 1) * L::LDD + 4 * v);
            }
            const float a[16] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w, cur[1].x, cur[1].y,
                                 cur[1].z, cur[1].w, cur[2].x, cur[2].y, cur[2].z, cur[2].w,
                                 cur[3].x, cur[3].y, cur[3].z, cur[3].w};
            const float xm = x[m];
#pragma unroll
            for (int r = m + 1; r < 16; ++r) x[r] = fmaf(-a[r], xm, x[r]);
#pragma unroll
            for (int v = 0; v < 4; ++v) cur[v] = nxt[v];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(16 * b + r) * LDT + 16 * b + c] = from_f<E>(x[r]);
        ptr.mark(3, wave, lane);
    } else if (wave == 1) {
        // blocks (1,0), (3,2), (0,1), (2,3) of T are read (as zeros) before they
        // are formed or as the upper triangle: 16 rows x 16 elements each
        const int blk = lane >> 4, r = lane & 15;
        const int br = (blk == 0) ? 1 : (blk == 1) ? 3 : (blk == 2) ? 0 : 2;
        const int bc = (blk == 0) ? 0 : (blk == 1) ? 2 : (blk == 2) ? 1 : 3;
        E *row = sT + (16 * br + r) * LDT + 16 * bc;
#pragma unroll
        for (int c = 0; c < 16; ++c) row[c] = from_f<E>(0.f);
    }
    lds_barrier();

    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // 3. T_10 and T_32 (wave 0: pair (1,0), wave 1: pair (3,2))
    if (wave < 2) {
        const int j = 2 * wave, i = j + 1;
        // X = A[i rows][16j .. 16j+31] T[16j .. 16j+31][j cols]; rows 16i.. of that
        // T range are T_ij, still zero, so X = A_ij T_jj
        const Frag<BF16> a = lds_frag<BF16>(sAe, LDT, 16 * i + cl, 16 * j, gq);
        const Frag<BF16> bt = lds_frag_tr<BF16>(sT, LDT, 16 * j, 16 * j, lane);
        const floatx4 X = mma(a, bt, zero4);
        // T_ij = -T[i rows][16j .. 16j+31] [0; X]  (= -T_ii X)
        const Frag<BF16> ti = lds_frag<BF16>(sT, LDT, 16 * i + cl, 16 * j, gq);
        const floatx4 Y = mma(ti, acc_frag<BF16>(zero4, X), zero4);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sT[(16 * i + 4 * gq + jj) * LDT + 16 * j + cl] = from_f<E>(-Y[jj]);
    }
    lds_barrier();

    ptr.mark(4, wave, lane);
    // 4. column tile j = wave of the lower-left 32x32 block
    if (wave < 2) {
        const int j = wave;
        const Frag<BF16> bt = lds_frag_tr<BF16>(sT, LDT, 0, 16 * j, lane);     // T[0..31][j cols]
        const floatx4 X2 = mma(lds_frag<BF16>(sAe, LDT, 32 + cl, 0, gq), bt, zero4);
        const floatx4 X3 = mma(lds_frag<BF16>(sAe, LDT, 48 + cl, 0, gq), bt, zero4);
        const Frag<BF16> bx = acc_frag<BF16>(X2, X3);                          // rows 32..63
        const floatx4 Y2 = mma(lds_frag<BF16>(sT, LDT, 32 + cl, 32, gq), bx, zero4);
        const floatx4 Y3 = mma(lds_frag<BF16>(sT, LDT, 48 + cl, 32, gq), bx, zero4);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            sT[(32 + 4 * gq + jj) * LDT + 16 * j + cl] = from_f<E>(-Y2[jj]);
            sT[(48 + 4 * gq + jj) * LDT + 16 * j + cl] = from_f<E>(-Y3[jj]);
        }
    }
    lds_barrier();

    ptr.mark(5, wave, lane);
    // 5. T as six fragment blocks.  Every entry of sT above the diagonal that a
    //    block covers is zero: the diagonal blocks' upper triangles come out of
    //    the substitution as zeros and blocks (0,1), (2,3) were cleared.
    constexpr int FB = kFragBytes<BF16>;
    for (int u = tid; u < 6 * 64; u += kPrepThreads) {
        const int b = u >> 6, p = u & 63;
        const int tt = b < 2 ? b : 2 + ((b - 2) >> 1), hh = b < 2 ? 0 : (b - 2) & 1;
        const int i = p >> 2, gg = (p & 3) ^ (i >> 2);
        const Frag<BF16> f = lds_frag<BF16>(sT, LDT, 16 * tt + i, 32 * hh, gg);
        uint4 w[FB / 16];
        __builtin_memcpy(w, &f, FB);
        uint4 *ub = reinterpret_cast<uint4 *>(dst + kWsT + b * kBlkBytes<BF16> + FB * p);
#pragma unroll
        for (int x = 0; x < FB / 16; ++x) ub[x] = w[x];
    }

    ptr.mark(6, wave, lane);
    // 6. LAG: R = T Y for row tiles tr of T (B operand: T's rows, k = rows of Y in
    //    fragment order; blocks of T above the diagonal are zero and skipped).  The
    //    accumulator of (tj = wave, tr) gives lane (g, i) R[16 tr + i][16 w + 4g + jj],
    //    half of the unit of block (tr, w / 2): elements 0..3 for even w, 4..7 for odd.
    if constexpr (LAG) {
        unsigned char *r1b = dst + WsLag::kR1, *r2b = dst + WsLag::kR2;
        const int off = 16 * blk_unit(cl, gq) + 8 * (wave & 1);
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                if (32 * hh > 16 * tr + 15) continue;
                const Frag<BF16> tf = lds_frag<BF16>(sT, LDT, 16 * tr + cl, 32 * hh, gq);
                a1 = mma(y1[hh], tf, a1);
                a2 = mma(y2[hh], tf, a2);
            }
            const int blk = 2 * tr + (wave >> 1);
            *reinterpret_cast<uint2 *>(r1b + blk * WsLag::kBlk + off) =
                make_uint2(pack2(a1[0], a1[1]), pack2(a1[2], a1[3]));
            *reinterpret_cast<uint2 *>(r2b + blk * WsLag::kBlk + off) =
                make_uint2(pack2(a2[0], a2[1]), pack2(a2[2], a2[3]));
        }
    }
}

// ---- the chunk-to-chunk scan -----------------------------------------------------
//
// One workgroup handles RW = 16 VT value rows of one (seq, head) and walks the
// chunks in order.  Value tile vt (16 rows) has three waves of its own:
//   X_vt  X = K M_n^T, E = beta (V - e^gam X), Delta = T E; publishes Delta (for
//         the output) and diag(e^{gam_last - gam}) Delta (for the update);
//   U_vt  holds its rows of M^T in fp32 and applies
//         M^T <- e^{gam_last} M^T + K^T (scaled Delta), publishing the new M^T
//         as B-operand fragment blocks;
//   O_vt  e^gam Q M_n^T / sqrt(d), then + (P / sqrt(d)) Delta: the output,
//         stored from registers;
// and four producer waves move the chunk data global -> LDS with
// global_load_lds (16 bytes per lane; a compute unit ingests faster the more
// waves keep such loads in flight).
//
// Two workgroup barriers per chunk n split the dependency chain between X and U,
// so that each one's LDS operand reads are done while the other computes:
//   A_n  M^T_n published                       X, O: products with M^T_n
//   B_n  Delta_n published                     U: state update; O: P Delta
// Between B_{n-1} and A_n, X reads its operands of chunk n into registers;
// between A_n and B_n, U reads its transposed K and O its Q and P of chunk n.
// Chunk data live in rings of SK (K, T, V, gates) and SQ (Q, P) slots, chunk m
// in slot m mod S.  The K/T slot of chunk m is read during [B_{m-1}, B_m) and
// refilled with chunk m+SK from B_m on; the Q/P slot is read during [A_m, B_m)
// and refilled with chunk m+SQ from A_{m+1} on.  A load thus has SK - 1 (SQ - 1)
// chunk steps to land, and the two kinds of loads are issued half a step apart.
// The fp32 variant (parity path) keeps one slot of each: a third barrier L_n per
// chunk marks the slot as loaded and the phases of a chunk run back to back.
//
// K and Q rows are padded by 32 bytes, which makes both the 16-byte row reads
// (k order 8g..8g+7 per lane group, matched by the key order of the published
// M^T blocks) and the transposing reads of K spread over the LDS banks.  T and
// P arrive as fragment blocks.  Rows past the end of a partial chunk are loaded
// from the last valid row: the prep kernel gives them beta = e^gam = 0, so they
// contribute nothing, and the data stay finite so that 0 * x = 0.

constexpr int kProducers = 4;

template <int D, bool BF16, int VT>
struct ScanCfg {
    static_assert(VT == 1 || VT == 2, "one or two value tiles per workgroup");
    using E = typename Elem<BF16>::T;
    static constexpr bool PIPE = BF16;
    static constexpr int RW = 16 * VT;              // value rows per workgroup
    static constexpr int ES = sizeof(E);
    static constexpr int KS = D / 32;
    static constexpr int FB = kFragBytes<BF16>;
    static constexpr int BLK = kBlkBytes<BF16>;
    // K, Q row stride (bytes): a multiple of 16 that is 2 mod 4 in 16-byte units, which
    // keeps both the 16-byte row reads and the transposing reads free of bank conflicts
    static constexpr int RK = D * ES + 32;
    static_assert((RK / 16) % 4 == 2, "K/Q row stride");
    static constexpr int RV = RW * ES + 16;         // V row stride
    // K/T/V/gates slot
    static constexpr int kK = 0;
    static constexpr int kT = kK + C * RK;
    static constexpr int kV = kT + 6 * BLK;
    static constexpr int kG = kV + C * RV;
    static constexpr int kSlotKT = kG + 2048;  // gates: one or two 1 KiB blocks
    // Q/P slot
    static constexpr int kQ = 0;
    static constexpr int kP = kQ + C * RK;
    static constexpr int kSlotQP = kP + 6 * BLK;
    // published values: M^T blocks, then Delta and scaled Delta as accumulator-pair
    // fragments
    static constexpr int kPubBytes = VT * KS * BLK + 4 * VT * 64 * FB;
    static constexpr int kLds = 160 * 1024;
    static constexpr bool fits(int sk, int sq) { return sk * kSlotKT + sq * kSlotQP + kPubBytes <= kLds; }
    static constexpr int SK = !PIPE ? 1 : fits(3, 2) ? 3 : 2;
    static constexpr int SQ = !PIPE ? 1 : fits(3, 3) ? 3 : 2;
    static constexpr int kRingKT = 0;
    static constexpr int kRingQP = kRingKT + SK * kSlotKT;
    static constexpr int kPubM = kRingQP + SQ * kSlotQP;
    static constexpr int kPubD = kPubM + VT * KS * BLK;
    static constexpr int kPubS = kPubD + 2 * VT * 64 * FB;
    static constexpr int kBytes = kPubS + 2 * VT * 64 * FB;
    static_assert(kBytes <= kLds, "LDS budget");
    // 1 KiB DMA blocks.  The regions of a slot are contiguous multiples of 1 KiB,
    // so block i of a slot's list lands at slot + 1024 i.
    static constexpr int NBK = C * RK / 1024;
    static constexpr int NBT = 6 * BLK / 1024;
    static constexpr int NBV = C * RV / 1024;
    static_assert(C * RK % 1024 == 0 && C * RV % 1024 == 0, "blocks");
    static constexpr int NKT = NBK + NBT + NBV + 1;  // K, T, V, gates (+1 gates block, NG)
    static constexpr int NQP = NBK + NBT;            // Q, P
    // producer p takes blocks p, p + 4, ...: its instruction counts; ng = 1 when
    // the second gates block (rows of normalised q/k) is loaded too
    static constexpr int nkt(int p, int ng) { return (NKT + ng + kProducers - 1 - p) / kProducers; }
    static constexpr int nqp(int p) { return (NQP + kProducers - 1 - p) / kProducers; }
    // Issue times (barrier A_j = time 2j, B_j = 2j + 1): right after A_j the
    // producers issue Q/P of chunk j + SQ - 1, right after B_j K/T of chunk j + SK;
    // the prologue issues the events of times t < 0 that have a chunk >= 0.
    static constexpr int qp_chunk(int t) { return t / 2 + SQ - 1; }          // t even
    static constexpr int kt_chunk(int t) { return (t - 1) / 2 + SK; }        // t odd
    // Number of a producer's load instructions issued at times in (lo, hi] for
    // chunks >= 0 (assuming every such chunk < n_chunks).
    static constexpr int issued(int lo, int hi, int p, int ng)
    {
        int c = 0;
        for (int t = lo + 1; t <= hi; ++t) {
            if (t % 2 == 0)
                c += qp_chunk(t) >= 0 ? nqp(p) : 0;
            else
                c += kt_chunk(t) >= 0 ? nkt(p, ng) : 0;
        }
        return c;
    }
    // Loads that may stay in flight at each wait, counted at n = 0 (a later n's
    // windows hold at least as many loads, so these counts stay safe):
    //   before B_{-1}: K/T of chunk 0 (issued at time 1 - 2 SK) has landed;
    //   before A_n:    Q/P of chunk n (issued at 2n + 2 - 2 SQ) has landed;
    //   before B_n:    K/T of chunk n+1 (issued at 2n + 3 - 2 SK) has landed.
    static constexpr int wait_prologue(int p, int ng) { return issued(1 - 2 * SK, -1, p, ng); }
    static constexpr int wait_a(int p, int ng) { return issued(2 - 2 * SQ, -1, p, ng); }
    static constexpr int wait_b(int p, int ng) { return issued(3 - 2 * SK, 0, p, ng); }
    static_assert(wait_prologue(0, 1) < 64 && wait_a(0, 1) < 64 && wait_b(0, 1) < 64,
                  "vmcnt range");
    static_assert(qp_chunk(2 - 2 * SQ) == 0 && kt_chunk(1 - 2 * SK) == 0, "issue times");
    static constexpr int kWaves = 3 * VT + kProducers;  // also in chunk_scan_kernel's launch bounds
};

// Workgroup barrier for the producer waves.  Their only LDS writes are the
// LDS-DMA loads, and a release fence would wait for every one of them to land
// (vmcnt 0), draining the prefetch pipeline at each barrier.  Instead each
// producer waits explicitly (wait_vmem_le) for exactly the loads that the
// barrier publishes; the loads still in flight write slots that no other wave
// reads before a later barrier.
__device__ __forceinline__ void dma_barrier() { __builtin_amdgcn_s_barrier(); }

struct ScanPtrs {
    const unsigned char *k, *q, *v;   // token 0 of this (seq, head); v at the first value row
    const unsigned char *ws;          // this (seq, head)'s chunk 0 in the workspace
    int64_t hd_bytes;                 // token stride of v in bytes (64 of them fit in 32 bits)
    int64_t kq_bytes;                 // token stride of k and q in bytes
    int64_t ws_stride;                // workspace bytes per chunk
};

// Producer PART's per-lane source offsets inside one chunk's data, for its K, T,
// V, gates blocks (kt) and its Q, P blocks (qp).  They depend on the chunk only
// through its number of valid rows, so they are formed once for full chunks and
// again for a partial last chunk, keeping that arithmetic out of the chunk loop
// (the producers share SIMDs with the waves on the dependency chain).
template <int D, bool BF16, int VT, int PART>
struct ProdOffsets {
    using F = ScanCfg<D, BF16, VT>;
    static constexpr int NK = (F::NKT + 1 - PART + kProducers - 1) / kProducers;
    static constexpr int NQ = (F::NQP - PART + kProducers - 1) / kProducers;
    uint32_t kt[NK], qp[NQ];

    __device__ __forceinline__ void set_kt(const ScanPtrs &pt, int nv, int lane)
    {
        const uint32_t hdb = static_cast<uint32_t>(pt.hd_bytes), kqb = static_cast<uint32_t>(pt.kq_bytes);
#pragma unroll
        for (int m = 0; m < NK; ++m) {
            const int i = PART + kProducers * m;
            if (i < F::NBK)
                kt[m] = dma_src_offset(i, lane, D * F::ES, F::RK, kqb, nv);
            else if (i < F::NBK + F::NBT)
                kt[m] = 1024u * (i - F::NBK) + 16u * lane;
            else if (i < F::NBK + F::NBT + F::NBV)
                kt[m] = dma_src_offset(i - F::NBK - F::NBT, lane, F::RW * F::ES, F::RV, hdb, nv);
            else
                kt[m] = 1024u * (i - F::NBK - F::NBT - F::NBV) + 16u * lane;
        }
    }
    __device__ __forceinline__ void set_qp(const ScanPtrs &pt, int nv, int lane)
    {
        const uint32_t kqb = static_cast<uint32_t>(pt.kq_bytes);
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int i = PART + kProducers * m;
            qp[m] = i < F::NBK ? dma_src_offset(i, lane, D * F::ES, F::RK, kqb, nv)
                               : 1024u * (i - F::NBK) + 16u * lane;
        }
    }
};

// Producer PART's blocks of chunk n's K, T, V and gates.
template <int D, bool BF16, int VT, int PART>
__device__ __forceinline__ void issue_kt(const ScanPtrs &pt, unsigned char *slot, int n, int ng,
                                        const ProdOffsets<D, BF16, VT, PART> &po)
{
    using F = ScanCfg<D, BF16, VT>;
    using W = WsLayout<BF16>;
    const int64_t tb = int64_t(n) * C * pt.hd_bytes, tbk = int64_t(n) * C * pt.kq_bytes;
    const unsigned char *wsc = pt.ws + int64_t(n) * pt.ws_stride;
#pragma unroll
    for (int i = PART; i < F::NKT + 1; i += kProducers) {
        if (i == F::NKT && !ng) break;
        const unsigned char *base;
        if (i < F::NBK)
            base = pt.k + tbk;
        else if (i < F::NBK + F::NBT)
            base = wsc + W::kT;
        else if (i < F::NBK + F::NBT + F::NBV)
            base = pt.v + tb;
        else
            base = wsc + W::kGates;
        dma16(base, po.kt[(i - PART) / kProducers], slot + 1024 * i);
    }
}

// Producer PART's blocks of chunk n's Q and P.
template <int D, bool BF16, int VT, int PART>
__device__ __forceinline__ void issue_qp(const ScanPtrs &pt, unsigned char *slot, int n,
                                        const ProdOffsets<D, BF16, VT, PART> &po)
{
    using F = ScanCfg<D, BF16, VT>;
    using W = WsLayout<BF16>;
    const int64_t tbk = int64_t(n) * C * pt.kq_bytes;
    const unsigned char *wsc = pt.ws + int64_t(n) * pt.ws_stride;
#pragma unroll
    for (int i = PART; i < F::NQP; i += kProducers)
        dma16(i < F::NBK ? pt.q + tbk : wsc + W::kP, po.qp[(i - PART) / kProducers], slot + 1024 * i);
}

// ---- wave roles ---------------------------------------------------------------

// X operands of one chunk.  The bf16 path holds the K and T fragments in
// registers (read before barrier A); the fp32 path reads them when used.
template <int D, bool BF16>
struct XOps {
    Frag<BF16> ak[4][D / 32];   // K rows: A operand of K M^T
    Frag<BF16> at[6];           // T blocks
    floatx4 be[4], edec[4];     // beta e^gam, e^{gam_last - gam}
    floatx4 bv[4];              // beta V for the tile's columns, accumulator layout
};

template <int D, bool BF16, int VT>
__device__ __forceinline__ void x_load(XOps<D, BF16> &o, const unsigned char *kt, int vt, int lane)
{
    using F = ScanCfg<D, BF16, VT>;
    const int gq = lane >> 4, cl = lane & 15;
    if constexpr (F::PIPE) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ks = 0; ks < F::KS; ++ks)
                o.ak[tt][ks] = row_frag<BF16>(kt + F::kK, F::RK, 16 * tt + cl, 32 * ks, gq);
#pragma unroll
        for (int b = 0; b < 6; ++b) o.at[b] = frag_blk<BF16>(kt + F::kT + b * F::BLK, lane);
    }
    const float *sG = reinterpret_cast<const float *>(kt + F::kG);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int t = 16 * tt + 4 * gq;
        const float4 b4 = *reinterpret_cast<const float4 *>(sG + t);
        const float4 e4 = *reinterpret_cast<const float4 *>(sG + C + t);
        const float4 d4 = *reinterpret_cast<const float4 *>(sG + 2 * C + t);
        const floatx4 bt = floatx4{b4.x, b4.y, b4.z, b4.w};
        o.be[tt] = bt * floatx4{e4.x, e4.y, e4.z, e4.w};
        o.edec[tt] = floatx4{d4.x, d4.y, d4.z, d4.w};
        o.bv[tt] = bt * col4<BF16>(kt + F::kV, F::RV, 16 * tt, 16 * vt, lane);
    }
}

// X_vt, one chunk (between barriers A and B): X = K M^T from the published M^T
// blocks, E = beta (V - e^gam X), Delta = T E; publishes Delta and
// diag(e^{gam_last - gam}) Delta.
template <int D, bool BF16, int VT>
__device__ __forceinline__ void x_step(const XOps<D, BF16> &o, const unsigned char *kt,
                                       unsigned char *smem, int vt, int lane)
{
    using F = ScanCfg<D, BF16, VT>;
    constexpr int KS = F::KS;
    const int gq = lane >> 4, cl = lane & 15;
    Frag<BF16> bm[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bm[ks] = frag_blk<BF16>(smem + F::kPubM + (vt * KS + ks) * F::BLK, lane);
    floatx4 xk[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) xk[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            if constexpr (F::PIPE)
                xk[tt] = mma(o.ak[tt][ks], bm[ks], xk[tt]);
            else
                xk[tt] = mma(row_frag<BF16>(kt + F::kK, F::RK, 16 * tt + cl, 32 * ks, gq), bm[ks],
                             xk[tt]);
        }
    floatx4 e[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) e[tt][j] = fmaf(-o.be[tt][j], xk[tt][j], o.bv[tt][j]);
    const Frag<BF16> be0 = acc_frag<BF16>(e[0], e[1]);
    const Frag<BF16> be1 = acc_frag<BF16>(e[2], e[3]);
    Frag<BF16> at[6];
#pragma unroll
    for (int b = 0; b < 6; ++b) {
        if constexpr (F::PIPE)
            at[b] = o.at[b];
        else
            at[b] = frag_blk<BF16>(kt + F::kT + b * F::BLK, lane);
    }
    floatx4 dl[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) dl[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
    tri_mul<BF16>(at, be0, be1, dl);
    floatx4 ds[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) ds[tt] = o.edec[tt] * dl[tt];
    Frag<BF16> *pS = reinterpret_cast<Frag<BF16> *>(smem + F::kPubS) + 128 * vt;
    Frag<BF16> *pD = reinterpret_cast<Frag<BF16> *>(smem + F::kPubD) + 128 * vt;
    pS[lane] = acc_frag<BF16>(ds[0], ds[1]);
    pS[64 + lane] = acc_frag<BF16>(ds[2], ds[3]);
    pD[lane] = acc_frag<BF16>(dl[0], dl[1]);
    pD[64 + lane] = acc_frag<BF16>(dl[2], dl[3]);
}

// U_vt: publishes its M^T tiles as fragment blocks with k (key) order 8g..8g+7.
// bf16: U's tiles hold keys in the permuted order of the whole-head pass (tile t,
// lane (gq, cl): keys 32 (t/2) + 8 gq + 4 (t%2) + 0..3), so tiles 2 ks and 2 ks + 1
// together are the lane's whole unit of block ks.  fp32: tile t holds keys
// 16t + 4gq + 0..3 and fills half of the units of block t/2.
template <int D, bool BF16, int VT>
__device__ __forceinline__ void publish_mt(const floatx4 (&Mt)[D / 16], unsigned char *smem, int vt,
                                           int lane)
{
    using F = ScanCfg<D, BF16, VT>;
    const int gq = lane >> 4, cl = lane & 15;
    if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < F::KS; ++ks)
            *reinterpret_cast<Frag<true> *>(smem + F::kPubM + (vt * F::KS + ks) * F::BLK +
                                            F::FB * blk_unit(cl, gq)) =
                acc_frag<true>(Mt[2 * ks], Mt[2 * ks + 1]);
    } else {
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            // lane (gq, cl) holds keys 16t + 4gq + 0..3: unit group 2 (t & 1) + gq / 2,
            // elements 4 (gq & 1) .. +3
            unsigned char *u = smem + F::kPubM + (vt * F::KS + (t >> 1)) * F::BLK +
                               F::FB * blk_unit(cl, 2 * (t & 1) + (gq >> 1)) + 4 * F::ES * (gq & 1);
            *reinterpret_cast<float4 *>(u) = make_float4(Mt[t][0], Mt[t][1], Mt[t][2], Mt[t][3]);
        }
    }
}

// Key of element j of U's state tile t in lane group gq (see publish_mt).
template <bool BF16>
__device__ __forceinline__ int u_key(int t, int gq)
{
    return BF16 ? 32 * (t >> 1) + 8 * gq + 4 * (t & 1) : 16 * t + 4 * gq;
}

// U_vt operands of one chunk (read between barriers A and B): K^T fragments
// (rows = key channels, k = tokens) and e^{gam_last}.
template <int D, bool BF16, int VT>
__device__ __forceinline__ void u_load(Frag<BF16> (&akt)[D / 16][2], float &eC,
                                       const unsigned char *kt, int lane)
{
    using F = ScanCfg<D, BF16, VT>;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
        if constexpr (BF16) {
            akt[t][0] = key_tr_frag(kt + F::kK, F::RK, 0, t, lane);
            akt[t][1] = key_tr_frag(kt + F::kK, F::RK, 32, t, lane);
        } else {
            akt[t][0] = frag_cols<BF16>(kt + F::kK, F::RK, 0, 16 * t, lane);
            akt[t][1] = frag_cols<BF16>(kt + F::kK, F::RK, 32, 16 * t, lane);
        }
    }
    eC = reinterpret_cast<const float *>(kt + F::kG)[3 * C];
}

// U_vt, one chunk (after barrier B): M^T <- M^T + K^T Dscaled, then publishes the
// new M^T.  The multiplication of M^T by e^{gam_last} is written before barrier B;
// the compiler interleaves it with these products, which measured faster than
// keeping it in the wait before the barrier.
template <int D, bool BF16, int VT>
__device__ __forceinline__ void u_step(floatx4 (&Mt)[D / 16], const Frag<BF16> (&akt)[D / 16][2],
                                       unsigned char *smem, int vt, int lane)
{
    using F = ScanCfg<D, BF16, VT>;
    const Frag<BF16> *pS = reinterpret_cast<const Frag<BF16> *>(smem + F::kPubS) + 128 * vt;
    const Frag<BF16> bs0 = pS[lane];
    const Frag<BF16> bs1 = pS[64 + lane];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) Mt[t] = mma(akt[t][0], bs0, Mt[t]);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) Mt[t] = mma(akt[t][1], bs1, Mt[t]);
    publish_mt<D, BF16, VT>(Mt, smem, vt, lane);
}

// O operands of one chunk.  The bf16 path holds the Q fragments in registers
// (read before barrier A); the fp32 path reads them when used.  P and the gates
// are always held: the slot may be refilled before they are used.
template <int D, bool BF16>
struct OOps {
    Frag<BF16> aq[4][D / 32];
    Frag<BF16> ap[6];
    float eg[4];                // e^gam / sqrt(d) of token 16 tt + lane % 16
};

template <int D, bool BF16, int VT>
__device__ __forceinline__ void o_load(OOps<D, BF16> &o, const unsigned char *kt,
                                       const unsigned char *qp, int eg_row, int lane)
{
    using F = ScanCfg<D, BF16, VT>;
    const int gq = lane >> 4, cl = lane & 15;
    if constexpr (F::PIPE) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ks = 0; ks < F::KS; ++ks)
                o.aq[tt][ks] = row_frag<BF16>(qp + F::kQ, F::RK, 16 * tt + cl, 32 * ks, gq);
    }
#pragma unroll
    for (int b = 0; b < 6; ++b) o.ap[b] = frag_blk<BF16>(qp + F::kP + b * F::BLK, lane);
    const float *sG = reinterpret_cast<const float *>(kt + F::kG);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) o.eg[tt] = kOutScale<D> * sG[eg_row * C + 16 * tt + cl];
}

// O_vt works on the transposed output tile, O^T = M Q^T diag(e^gam) + Delta^T P^T
// (1/sqrt(d) already in e^gam and P):
// an A operand and a B operand of the same matrix have the same register layout, so
// the products are those of O with their operands swapped, and the accumulator of
// row tile tt holds in lane (g, i) the values 4g .. 4g+3 of token 16 tt + i, which
// is stored from registers as it stands.
//
// O_vt between barriers A and B: acc = (e^gam (Q M^T))^T.
template <int D, bool BF16, int VT>
__device__ __forceinline__ void o_xq(const OOps<D, BF16> &o, const unsigned char *qp,
                                     const unsigned char *smem, int vt, int lane, floatx4 (&acc)[4])
{
    using F = ScanCfg<D, BF16, VT>;
    constexpr int KS = F::KS;
    const int gq = lane >> 4, cl = lane & 15;
    Frag<BF16> bm[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bm[ks] = frag_blk<BF16>(smem + F::kPubM + (vt * KS + ks) * F::BLK, lane);
    floatx4 xq[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) xq[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            if constexpr (F::PIPE)
                xq[tt] = mma(bm[ks], o.aq[tt][ks], xq[tt]);
            else
                xq[tt] = mma(bm[ks], row_frag<BF16>(qp + F::kQ, F::RK, 16 * tt + cl, 32 * ks, gq),
                             xq[tt]);
        }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = xq[tt] * o.eg[tt];
}

// O_vt after barrier B: acc += (P Delta)^T, which is the output of the valid
// tokens, stored from registers (four consecutive values of one token per lane and
// row tile; no per-token test for a full chunk).  obase points at out[(s, first
// token of the chunk, h, first value row of the tile)].
template <int D, bool BF16, int VT>
__device__ __forceinline__ void o_finish(const OOps<D, BF16> &o, const unsigned char *smem, int vt,
                                         int lane, floatx4 (&acc)[4], typename Elem<BF16>::T *obase,
                                         int64_t hd, int nv)
{
    using F = ScanCfg<D, BF16, VT>;
    const int gq = lane >> 4, cl = lane & 15;
    const Frag<BF16> *pD = reinterpret_cast<const Frag<BF16> *>(smem + F::kPubD) + 128 * vt;
    const Frag<BF16> d0 = pD[lane];
    const Frag<BF16> d1 = pD[64 + lane];
    acc[0] = mma(d0, o.ap[0], acc[0]);
    acc[1] = mma(d0, o.ap[1], acc[1]);
    acc[2] = mma(d1, o.ap[3], mma(d0, o.ap[2], acc[2]));
    acc[3] = mma(d1, o.ap[5], mma(d0, o.ap[4], acc[3]));
    auto store = [&](int tt) {
        typename Elem<BF16>::T *dst = obase + (16 * tt + cl) * hd + 4 * gq;
        if constexpr (BF16)
            *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2(acc[tt][0], acc[tt][1]),
                                                         pack2(acc[tt][2], acc[tt][3]));
        else
            *reinterpret_cast<float4 *>(dst) = make_float4(acc[tt][0], acc[tt][1], acc[tt][2],
                                                           acc[tt][3]);
    };
    if (nv == C) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) store(tt);
    } else {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
            if (16 * tt + cl < nv) store(tt);
    }
}

// Producer PART: moves every chunk's data into its ring slots and waits for it
// before the barrier after which it is read.
template <int D, bool BF16, int VT, int PART, int NG>
__device__ __forceinline__ void producer_loop(const ScanPtrs &pt, unsigned char *smem, int nc,
                                              int64_t n_tokens, int lane)
{
    using F = ScanCfg<D, BF16, VT>;
    constexpr int SK = F::SK, SQ = F::SQ;
    auto nv_of = [&](int m) { return static_cast<int>(min<int64_t>(C, n_tokens - int64_t(m) * C)); };
    // offsets for full chunks; a partial chunk is the last one of each kind issued
    ProdOffsets<D, BF16, VT, PART> po;
    po.set_kt(pt, C, lane);
    po.set_qp(pt, C, lane);
    auto kt = [&](int m) {
        if (m < nc) {
            if (nv_of(m) < C) po.set_kt(pt, nv_of(m), lane);
            issue_kt<D, BF16, VT, PART>(pt, smem + F::kRingKT + (m % SK) * F::kSlotKT, m, NG, po);
        }
    };
    auto qp = [&](int m) {
        if (m < nc) {
            if (nv_of(m) < C) po.set_qp(pt, nv_of(m), lane);
            issue_qp<D, BF16, VT, PART>(pt, smem + F::kRingQP + (m % SQ) * F::kSlotQP, m, po);
        }
    };
    if constexpr (F::PIPE) {
        // prologue: the issues of times t < 0, oldest first
#pragma unroll
        for (int t = (2 - 2 * SQ < 1 - 2 * SK ? 2 - 2 * SQ : 1 - 2 * SK); t < 0; ++t) {
            if (t % 2 == 0) {
                if (F::qp_chunk(t) >= 0) qp(F::qp_chunk(t));
            } else if (F::kt_chunk(t) >= 0) {
                kt(F::kt_chunk(t));
            }
        }
        constexpr int SM = SK > SQ ? SK : SQ;
        if (nc >= SM)
            wait_vmem_le<F::wait_prologue(PART, NG)>();
        else
            wait_vmem_le<0>();
        dma_barrier();  // B_{-1}: K/T of chunk 0 is in LDS
        for (int n = 0; n < nc; ++n) {
            // near the end some of the counted loads were never issued: wait for all
            if (n + SM < nc)
                wait_vmem_le<F::wait_a(PART, NG)>();  // Q/P of chunk n landed
            else
                wait_vmem_le<0>();
            dma_barrier();  // A_n: Q/P slot of chunk n-1 is free
            qp(n + SQ - 1);
            if (n + SM < nc)
                wait_vmem_le<F::wait_b(PART, NG)>();  // K/T of chunk n+1 landed
            else
                wait_vmem_le<0>();
            dma_barrier();  // B_n: K/T slot of chunk n is free
            kt(n + SK);
        }
    } else {
        for (int n = 0; n < nc; ++n) {
            kt(n);
            qp(n);
            wait_vmem_le<0>();
            dma_barrier();  // L_n
            dma_barrier();  // A_n
            dma_barrier();  // B_n
        }
    }
}

// Per-tile pass timestamps (trace builds only): for waves X_0, U_0, O_0 and each
// chunk, arriving at and leaving barrier A (slots 0, 1), arriving at and leaving
// barrier B (slots 2, 3); row [3][0] holds the workgroup's edges: X_0 starting,
// X_0 leaving the first barrier, U_0 done storing the state, O_0 done storing the
// last output; gdn_scan_trace_read copies them out.
#ifdef GDN_PHASE_TRACE
__device__ uint64_t g_scan_trace[kTraceGroups][4][kTracePhases][4];
// every workgroup's X_0 start, U_0 end and O_0 end on the chip-wide 100 MHz clock
constexpr int kSpanGroups = 4096;
__device__ uint64_t g_scan_span[kSpanGroups][4];
#endif

struct ScanTrace {
    int64_t wg;
    int role;      // 0 X, 1 U, 2 O; waves of value tile 0 only
    __device__ __forceinline__ void mark(int n, int slot, int lane) const
    {
#ifdef GDN_PHASE_TRACE
        if (wg < kTraceGroups && role >= 0 && lane == 0 && n < kTracePhases)
            g_scan_trace[wg][role][n][slot] = __builtin_amdgcn_s_memtime();
#else
        (void)n;
        (void)slot;
        (void)lane;
#endif
    }
    __device__ __forceinline__ void edge(int which, int lane) const
    {
#ifdef GDN_PHASE_TRACE
        if (which >= 2) __builtin_amdgcn_s_waitcnt(0);  // the stores have left the wave
        if (wg < kTraceGroups && role >= 0 && lane == 0)
            g_scan_trace[wg][3][0][which] = __builtin_amdgcn_s_memtime();
        if (wg < kSpanGroups && role >= 0 && lane == 0 && which != 1)
            g_scan_span[wg][which == 0 ? 0 : which - 1] = __builtin_amdgcn_s_memrealtime();
#else
        (void)which;
        (void)lane;
#endif
    }
};

enum { kRoleX = 0, kRoleU = 1, kRoleO = 2, kRoleProd = 3 };

// Wave order: X_0.., U_0.., then O and the producers arranged so that, with
// waves dealt round-robin to the four SIMDs, no O wave shares a SIMD with an X
// wave (both run their products between barriers A and B).
template <int VT>
__device__ __forceinline__ void wave_role(int wave, int &role, int &idx)
{
    if (wave < 2 * VT) {
        role = wave / VT;
        idx = wave % VT;
    } else if constexpr (VT == 1) {
        role = wave == 2 ? kRoleO : kRoleProd;  // 2: O; 3..6: producers
        idx = wave == 2 ? 0 : wave - 3;
    } else {
        // 4, 5: producers 0, 1; 6, 7: O_0, O_1; 8, 9: producers 2, 3
        role = (wave == 6 || wave == 7) ? kRoleO : kRoleProd;
        idx = wave < 6 ? wave - 4 : wave - 6;
    }
}

// Workgroups are numbered so that the row blocks of one (seq, head) share the
// low three bits of the block id: consecutive ids go to different XCDs, so this
// keeps a head's workgroups on one XCD, where its K, Q, T and P hit in L2.
template <int D, bool BF16, int VT, bool NORM>
__global__ __launch_bounds__(64 * (3 * VT + kProducers)) void chunk_scan_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *state_in, void *__restrict__ out, float *state_out,
    const unsigned char *__restrict__ ws, int64_t n_tokens, int64_t n_heads, int64_t n_k_heads,
    int64_t n_sh, int n_chunks)
{
    using F = ScanCfg<D, BF16, VT>;
    using E = typename Elem<BF16>::T;
    using W = WsLayout<BF16>;
    constexpr int NRB = D / F::RW;  // row blocks per head
    constexpr bool PIPE = F::PIPE;
    extern __shared__ __align__(16) unsigned char smem[];

    const int64_t b = blockIdx.x;
    const int64_t sh = (b / (8 * NRB)) * 8 + (b & 7);
    const int rb = static_cast<int>((b >> 3) % NRB);
    if (sh >= n_sh) return;  // whole workgroup leaves before any barrier
    const int64_t s = sh / n_heads, h = sh - s * n_heads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int v0 = rb * F::RW;                       // first value row of the workgroup
    const int64_t hd = n_heads * D;
    const int64_t tok0 = (s * n_tokens * n_heads + h) * D;                        // v, out
    const int64_t ktok0 = (s * n_tokens * n_k_heads + h % n_k_heads) * D;         // k, q
    const int nc = n_chunks;
    auto nv_of = [&](int n) { return static_cast<int>(min<int64_t>(C, n_tokens - int64_t(n) * C)); };
    auto kt_slot = [&](int n) { return smem + F::kRingKT + (n % F::SK) * F::kSlotKT; };
    auto qp_slot = [&](int n) { return smem + F::kRingQP + (n % F::SQ) * F::kSlotQP; };

    int role, vt;
    wave_role<VT>(wave, role, vt);
    if (role == kRoleProd) {
        ScanPtrs pt;
        pt.k = static_cast<const unsigned char *>(k) + ktok0 * F::ES;
        pt.q = static_cast<const unsigned char *>(q) + ktok0 * F::ES;
        pt.v = static_cast<const unsigned char *>(v) + (tok0 + v0) * F::ES;
        pt.ws_stride = W::stride(NORM);
        pt.ws = ws + sh * nc * pt.ws_stride;
        pt.hd_bytes = hd * F::ES;
        pt.kq_bytes = n_k_heads * D * F::ES;
        // the second gates block (e^gam / |q|) is loaded only for normalised rows
        if constexpr (NORM) {
            switch (vt) {
            case 0: producer_loop<D, BF16, VT, 0, 1>(pt, smem, nc, n_tokens, lane); break;
            case 1: producer_loop<D, BF16, VT, 1, 1>(pt, smem, nc, n_tokens, lane); break;
            case 2: producer_loop<D, BF16, VT, 2, 1>(pt, smem, nc, n_tokens, lane); break;
            default: producer_loop<D, BF16, VT, 3, 1>(pt, smem, nc, n_tokens, lane); break;
            }
        } else {
            switch (vt) {
            case 0: producer_loop<D, BF16, VT, 0, 0>(pt, smem, nc, n_tokens, lane); break;
            case 1: producer_loop<D, BF16, VT, 1, 0>(pt, smem, nc, n_tokens, lane); break;
            case 2: producer_loop<D, BF16, VT, 2, 0>(pt, smem, nc, n_tokens, lane); break;
            default: producer_loop<D, BF16, VT, 3, 0>(pt, smem, nc, n_tokens, lane); break;
            }
        }
        return;
    }

    const ScanTrace tr{b, (vt == 0 && role != kRoleProd && PIPE) ? role : -1};
    if (role == kRoleX) {
        XOps<D, BF16> ops;
        tr.edge(0, lane);
        if constexpr (PIPE) lds_barrier();  // B_{-1}
        tr.edge(1, lane);
        for (int n = 0; n < nc; ++n) {
            if constexpr (!PIPE) lds_barrier();  // L_n
            x_load<D, BF16, VT>(ops, kt_slot(n), vt, lane);
            tr.mark(n, 0, lane);
            lds_barrier();  // A_n
            tr.mark(n, 1, lane);
            x_step<D, BF16, VT>(ops, kt_slot(n), smem, vt, lane);
            tr.mark(n, 2, lane);
            lds_barrier();  // B_n
            tr.mark(n, 3, lane);
        }
    } else if (role == kRoleU) {
        // Mt[t][j] = M[v0 + 16 vt + lane%16][u_key(t, lane/16) + j]
        const int64_t st_off = sh * D * D + int64_t(v0 + 16 * vt + (lane & 15)) * D;
        floatx4 Mt[D / 16];
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            if (state_in) {
                const float4 m = *reinterpret_cast<const float4 *>(state_in + st_off + u_key<BF16>(t, lane >> 4));
                Mt[t] = floatx4{m.x, m.y, m.z, m.w};
            } else {
                Mt[t] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        }
        publish_mt<D, BF16, VT>(Mt, smem, vt, lane);
        Frag<BF16> akt[D / 16][2];
        float eC;
        if constexpr (PIPE) lds_barrier();  // B_{-1}
        for (int n = 0; n < nc; ++n) {
            if constexpr (!PIPE) lds_barrier();  // L_n
            tr.mark(n, 0, lane);
            lds_barrier();  // A_n
            tr.mark(n, 1, lane);
            u_load<D, BF16, VT>(akt, eC, kt_slot(n), lane);
#pragma unroll
            for (int t = 0; t < D / 16; ++t) Mt[t] *= eC;
            tr.mark(n, 2, lane);
            lds_barrier();  // B_n
            tr.mark(n, 3, lane);
            u_step<D, BF16, VT>(Mt, akt, smem, vt, lane);
        }
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
            *reinterpret_cast<float4 *>(state_out + st_off + u_key<BF16>(t, lane >> 4)) =
                make_float4(Mt[t][0], Mt[t][1], Mt[t][2], Mt[t][3]);
        tr.edge(2, lane);
    } else {
        E *obase = static_cast<E *>(out) + tok0 + v0 + 16 * vt;
        constexpr int eg_row = NORM ? 4 : 1;  // e^gam, or e^gam / |q| for normalised rows
        OOps<D, BF16> ops;
        floatx4 acc[4];
        if constexpr (PIPE) lds_barrier();  // B_{-1}
        for (int n = 0; n < nc; ++n) {
            if constexpr (!PIPE) lds_barrier();  // L_n
            tr.mark(n, 0, lane);
            lds_barrier();  // A_n
            tr.mark(n, 1, lane);
            o_load<D, BF16, VT>(ops, kt_slot(n), qp_slot(n), eg_row, lane);
            o_xq<D, BF16, VT>(ops, qp_slot(n), smem, vt, lane, acc);
            tr.mark(n, 2, lane);
            lds_barrier();  // B_n
            tr.mark(n, 3, lane);
            o_finish<D, BF16, VT>(ops, smem, vt, lane, acc, obase + int64_t(n) * C * hd, hd,
                                  nv_of(n));
        }
        tr.edge(3, lane);
    }
}

template <int D, bool BF16, bool NORM, bool LAG, bool PQ = true>
hipError_t launch_prep(const Problem &p, unsigned char *ws, int n_chunks, hipStream_t stream)
{
    using L = PrepSmem<D, BF16>;
    auto kern = chunk_prep_kernel<D, BF16, NORM, LAG, PQ>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = ensure_lds_limit(kern, L::kBytes, lds_set);
    if (e != hipSuccess) return e;
    const int64_t blocks = p.n_seqs * p.n_heads * n_chunks;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(kPrepThreads), L::kBytes,
                       stream, p.q, p.k, p.g, p.beta, ws, p.n_tokens, p.n_heads, p.n_k_heads,
                       n_chunks, p.raw_gates);
    return hipGetLastError();
}

// Scan workgroups: the row blocks of every (seq, head), heads padded to a multiple
// of eight (one XCD per head).
template <int D, bool BF16, int VT>
int64_t scan_blocks(int64_t n_sh)
{
    return (n_sh + 7) / 8 * 8 * (D / ScanCfg<D, BF16, VT>::RW);
}

template <int D, bool BF16, int VT, bool NORM>
hipError_t launch_scan(const Problem &p, const unsigned char *ws, int n_chunks, hipStream_t stream)
{
    using F = ScanCfg<D, BF16, VT>;
    auto kern = chunk_scan_kernel<D, BF16, VT, NORM>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = ensure_lds_limit(kern, F::kBytes, lds_set);
    if (e != hipSuccess) return e;
    const int64_t n_sh = p.n_seqs * p.n_heads;
    const int64_t blocks = scan_blocks<D, BF16, VT>(n_sh);
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(64 * F::kWaves), F::kBytes,
                       stream, p.q, p.k, p.v, p.state_in, p.out, p.state_out, ws, p.n_tokens,
                       p.n_heads, p.n_k_heads, n_sh, n_chunks);
    return hipGetLastError();
}

// Compute units of the current device (looked up once per device).
int cu_count()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// The prep, then the chunk-to-chunk pass.  The whole-head pass (bf16) when forced,
// or under AUTO from one (seq, head) per compute unit on; else the two-barrier
// scan, for bf16 with two value tiles per workgroup once one tile each would give
// more workgroups than compute units; fp32 keeps one tile and one ring slot.  lag
// (bf16 only): the prep with the lag form's cross-chunk matrices, then the lag scan.
// Normalised q/k rows are a prep (and two-barrier scan) variant of their own (NORM),
// so that the plain kernels carry none of that mode's code; the lag scan reads the
// normalisation through the gate rows and has no such variant.
template <int D, bool BF16, bool NORM>
hipError_t launch_chunk_dn(const Problem &p, bool lag, unsigned char *ws, hipStream_t stream)
{
    if constexpr (BF16) {
        // the whole-head scan when forced, or (unless the lag form is asked for) once
        // there is a (seq, head) for every compute unit: each workgroup then brings
        // a chunk's shared operands in once for all value rows
        const bool head = p.head_scan > 0 ||
                          (p.head_scan == 0 && !lag && p.n_seqs * p.n_heads >= cu_count());
        if (head) {
            const int64_t n_chunks64 = (p.n_tokens + C - 1) / C;
            const int64_t n_sh = p.n_seqs * p.n_heads;
            if (n_chunks64 > INT32_MAX || !grid_fits(n_sh * n_chunks64, kPrepThreads) ||
                !head_pass_fits(n_sh, D))
                return hipErrorInvalidConfiguration;
            const int n_chunks = static_cast<int>(n_chunks64);
            // plain rows: the pass forms P itself, and the prep skips Q
            const hipError_t e = NORM ? launch_prep<D, BF16, NORM, false>(p, ws, n_chunks, stream)
                                      : launch_prep<D, BF16, false, false, false>(p, ws, n_chunks,
                                                                                  stream);
            return e != hipSuccess ? e : launch_head_pass(p, ws, n_chunks, stream);
        }
    }
    const int64_t n_chunks64 = (p.n_tokens + C - 1) / C;
    const int64_t n_sh = p.n_seqs * p.n_heads;
    const bool vt1 = !BF16 || n_sh * (D / 16) <= 256;
    // both grids are checked before either kernel is launched
    const bool scan_fits =
        lag ? lag_pass_fits(n_sh, D)
        : vt1 ? grid_fits(scan_blocks<D, BF16, 1>(n_sh), 64 * ScanCfg<D, BF16, 1>::kWaves)
              : grid_fits(scan_blocks<D, BF16, 2>(n_sh), 64 * ScanCfg<D, BF16, 2>::kWaves);
    if (n_chunks64 > INT32_MAX || !grid_fits(n_sh * n_chunks64, kPrepThreads) || !scan_fits)
        return hipErrorInvalidConfiguration;
    const int n_chunks = static_cast<int>(n_chunks64);
    if constexpr (BF16) {
        if (lag) {
            const hipError_t e = launch_prep<D, BF16, NORM, true>(p, ws, n_chunks, stream);
            return e != hipSuccess ? e : launch_lag_pass(p, ws, n_chunks, stream);
        }
    } else if (lag) {
        return hipErrorInvalidValue;   // refused by the API before this point
    }
    const hipError_t e = launch_prep<D, BF16, NORM, false>(p, ws, n_chunks, stream);
    if (e != hipSuccess) return e;
    if (vt1) return launch_scan<D, BF16, 1, NORM>(p, ws, n_chunks, stream);
    if constexpr (BF16) return launch_scan<D, BF16, 2, NORM>(p, ws, n_chunks, stream);
    return hipErrorInvalidValue;  // not reached
}

template <int D, bool BF16>
hipError_t launch_chunk_d(const Problem &p, bool lag, unsigned char *ws, hipStream_t stream)
{
    return p.l2norm_qk ? launch_chunk_dn<D, BF16, true>(p, lag, ws, stream)
                       : launch_chunk_dn<D, BF16, false>(p, lag, ws, stream);
}

template <bool BF16>
hipError_t launch_chunk_t(const Problem &p, bool lag, unsigned char *ws, hipStream_t stream)
{
    switch (p.head_dim) {
    case 32: return launch_chunk_d<32, BF16>(p, lag, ws, stream);
    case 64: return launch_chunk_d<64, BF16>(p, lag, ws, stream);
    case 96: return launch_chunk_d<96, BF16>(p, lag, ws, stream);
    case 128: return launch_chunk_d<128, BF16>(p, lag, ws, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t chunk_workspace_bytes(int bf16, int lag, int64_t n_seqs, int64_t n_tokens,
                             int64_t n_heads, int)
{
    const int64_t n_chunks = (n_tokens + C - 1) / C;
    // the lag form's layout, else sized for the larger (normalised q/k) layout, so
    // one workspace serves both
    const int64_t per = (bf16 && lag) ? WsLag::kBytes
                        : bf16        ? WsLayout<true>::kBytesNorm
                                      : WsLayout<false>::kBytesNorm;
    return static_cast<size_t>(n_seqs * n_heads * n_chunks * per);
}

#ifdef GDN_PHASE_TRACE
// Copies the timestamps of the last prep out (trace builds only; not part of the
// installed interface).
extern "C" int gdn_prep_trace_read(void *host, size_t bytes)
{
    if (bytes > sizeof(g_prep_trace)) bytes = sizeof(g_prep_trace);
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_prep_trace), bytes, 0, hipMemcpyDeviceToHost) ==
                   hipSuccess
               ? 0
               : -1;
}

// Copies every workgroup's start and end stamps of the last per-tile pass out (trace
// builds only; not part of the installed interface).
extern "C" int gdn_scan_span_read(void *host, size_t bytes)
{
    if (bytes > sizeof(g_scan_span)) bytes = sizeof(g_scan_span);
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_scan_span), bytes, 0, hipMemcpyDeviceToHost) ==
                   hipSuccess
               ? 0
               : -1;
}

// Copies the timestamps of the last per-tile pass out (trace builds only; not part
// of the installed interface).
extern "C" int gdn_scan_trace_read(void *host, size_t bytes)
{
    if (bytes > sizeof(g_scan_trace)) bytes = sizeof(g_scan_trace);
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_scan_trace), bytes, 0, hipMemcpyDeviceToHost) ==
                   hipSuccess
               ? 0
               : -1;
}
#endif

hipError_t launch_chunked(const Problem &p, bool lag, void *workspace, hipStream_t stream)
{
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    return p.bf16 ? launch_chunk_t<true>(p, lag, ws, stream)
                  : launch_chunk_t<false>(p, lag, ws, stream);
}

}  // namespace gdn
