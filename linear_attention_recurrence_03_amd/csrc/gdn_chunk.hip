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
// Two kernels:
//   chunk_prep_kernel  -- one workgroup per (seq, head, chunk), all chunks in
//                         parallel: the state-independent part (gates, A, T, P).
//                         K K^T and Q K^T run on MFMA; T comes from a blocked
//                         triangular inverse in LDS (16x16 diagonal blocks by
//                         forward substitution, then the off-diagonal blocks).
//                         Writes T, P and the gate vectors to the workspace.
//   chunk_scan_kernel  -- one workgroup per (seq, head, block of value rows),
//                         walking the chunks in order and carrying its rows of
//                         M in registers.  Value rows of M are independent given
//                         k, q, g, beta, so splitting them across workgroups
//                         needs no communication.  Each wave owns 16 value rows
//                         and does K M^T, Q M^T, T E, P Delta and the state
//                         update on MFMA (16x16x32 bf16 for bf16 inputs,
//                         16x16x4 fp32 for fp32 inputs), with the chunk's K, K^T,
//                         Q, T, P and V staged in LDS; the next chunk's loads
//                         are in flight while the current one is computed.
//
// MFMA fragments.  An A operand (16 rows x 32 k) gives lane l row l%16 and eight
// k values; a B operand (32 k x 16 cols) gives lane l column l%16 and eight k
// values; the hardware pairs element j of lane group g = l/16 in A with the same
// element of B.  The accumulator gives lane l column l%16 and rows 4g..4g+3.
// Two stacked accumulator tiles therefore form a B operand directly if element
// j of group g stands for row 4g+j (j < 4) or 16+4g+j-4 (j >= 4) of the 32; every
// A operand here is loaded with that same k order, so no data moves between
// lanes when a product feeds the next one.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int C = kChunk;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
    using T = uint16_t;
};
template <>
struct Elem<false> {
    using T = float;
};

__device__ __forceinline__ float to_f(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f(float x) { return x; }
template <class T>
__device__ __forceinline__ T from_f(float x);
template <>
__device__ __forceinline__ uint16_t from_f<uint16_t>(float x)
{
    return f32_to_bf16(x);
}
template <>
__device__ __forceinline__ float from_f<float>(float x)
{
    return x;
}

// ---- fragments ---------------------------------------------------------------

template <bool BF16>
struct Frag;
template <>
struct Frag<true> {
    uint4 u;  // eight bf16
};
template <>
struct Frag<false> {
    float v[8];
};

__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// k order of a fragment: element j of lane group g is k = 4g+j (j<4), 16+4g+j-4.
// Row `row` of a row-major LDS matrix with leading dimension ld, k offset k0.
template <bool BF16>
__device__ __forceinline__ Frag<BF16> lds_frag(const typename Elem<BF16>::T *base, int ld, int row,
                                               int k0, int g)
{
    Frag<BF16> f;
    const typename Elem<BF16>::T *p = base + row * ld + k0 + 4 * g;
    if constexpr (BF16) {
        const uint2 lo = *reinterpret_cast<const uint2 *>(p);
        const uint2 hi = *reinterpret_cast<const uint2 *>(p + 16);
        f.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
        const float4 lo = *reinterpret_cast<const float4 *>(p);
        const float4 hi = *reinterpret_cast<const float4 *>(p + 16);
        f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
        f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
    }
    return f;
}

// B operand from two stacked accumulator tiles, element-wise scaled by s0/s1.
template <bool BF16>
__device__ __forceinline__ Frag<BF16> acc_frag(const floatx4 &c0, const floatx4 &c1)
{
    Frag<BF16> f;
    if constexpr (BF16) {
        f.u = make_uint4(pack2(c0[0], c0[1]), pack2(c0[2], c0[3]), pack2(c1[0], c1[1]),
                         pack2(c1[2], c1[3]));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f.v[j] = c0[j];
            f.v[4 + j] = c1[j];
        }
    }
    return f;
}

__device__ __forceinline__ floatx4 mma(const Frag<true> &a, const Frag<true> &b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.u),
                                                   __builtin_bit_cast(bf16x8_t, b.u), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mma(const Frag<false> &a, const Frag<false> &b, floatx4 c)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
}

// ---- workspace layout, per (seq, head, chunk) ----------------------------------
//   T     [C][C] elements   (fp32 or bf16, like q/k/v)
//   P     [C][C] elements
//   gates [C][4] fp32: per token r {beta_r, e^{gam_r}, e^{gam_last - gam_r},
//                      e^{gam_last}}
// Rows past the end of a partial last chunk carry beta = e^gam = 0, so they add
// nothing to the state or to valid outputs.
template <bool BF16>
struct WsLayout {
    using E = typename Elem<BF16>::T;
    static constexpr int64_t kT = 0;
    static constexpr int64_t kP = int64_t(C) * C * sizeof(E);
    static constexpr int64_t kGates = 2 * kP;
    static constexpr int64_t kBytes = kGates + 4 * C * 4;
};

constexpr int kPrepThreads = 256;

template <int D, bool BF16>
struct PrepSmem {
    using E = typename Elem<BF16>::T;
    static constexpr int LDK = D + (BF16 ? 8 : 4);  // padded row, elements
    static constexpr int LDA = C + 1;               // fp32 square matrices
    static constexpr int kK = 0;
    static constexpr int kQ = kK + C * LDK * sizeof(E);
    static constexpr int kA = kQ + C * LDK * sizeof(E);
    static constexpr int kT = kA + C * LDA * 4;
    static constexpr int kP = kT + C * LDA * 4;
    static constexpr int kX = kP + C * LDA * 4;  // 3 blocks of 16x17 fp32
    static constexpr int kG = kX + 3 * 16 * 17 * 4;
    static constexpr int kBytes = kG + (4 * C + 4) * 4;
};

// Lower 16x16 tiles (tr >= tc) of a 4x4 tile grid, in a fixed order.
__device__ __forceinline__ void lower_tile(int ix, int &tr, int &tc)
{
    tr = (ix >= 6) ? 3 : (ix >= 3) ? 2 : (ix >= 1) ? 1 : 0;
    tc = ix - tr * (tr + 1) / 2;
}

template <int D, bool BF16>
__global__ __launch_bounds__(kPrepThreads) void chunk_prep_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, unsigned char *__restrict__ ws, int64_t n_tokens,
    int64_t n_heads, int n_chunks)
{
    using E = typename Elem<BF16>::T;
    using L = PrepSmem<D, BF16>;
    using W = WsLayout<BF16>;
    constexpr int LDK = L::LDK, LDA = L::LDA;
    extern __shared__ __align__(16) unsigned char smem[];
    E *sK = reinterpret_cast<E *>(smem + L::kK);
    E *sQ = reinterpret_cast<E *>(smem + L::kQ);
    float *sA = reinterpret_cast<float *>(smem + L::kA);
    float *sT = reinterpret_cast<float *>(smem + L::kT);
    float *sP = reinterpret_cast<float *>(smem + L::kP);
    float *sX = reinterpret_cast<float *>(smem + L::kX);
    float *sG = reinterpret_cast<float *>(smem + L::kG);  // gam, beta, e^gam, e^{last-gam}, e^last

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t chunk_id = blockIdx.x;
    const int64_t sh = chunk_id / n_chunks;
    const int n = static_cast<int>(chunk_id - sh * n_chunks);
    const int64_t s = sh / n_heads, h = sh - s * n_heads;
    const int64_t t0 = int64_t(n) * C;
    const int nv = static_cast<int>(min<int64_t>(C, n_tokens - t0));

    // 1. K and Q rows of the chunk (zero past the end of the sequence)
    constexpr int VE = 16 / sizeof(E);
    constexpr int VPR = D / VE;
    for (int i = tid; i < C * VPR; i += kPrepThreads) {
        const int r = i / VPR, c = (i - r * VPR) * VE;
        uint4 kv = make_uint4(0, 0, 0, 0), qv = kv;
        if (r < nv) {
            const int64_t off = ((s * n_tokens + t0 + r) * n_heads + h) * D + c;
            kv = *reinterpret_cast<const uint4 *>(static_cast<const E *>(k) + off);
            qv = *reinterpret_cast<const uint4 *>(static_cast<const E *>(q) + off);
        }
        *reinterpret_cast<uint4 *>(sK + r * LDK + c) = kv;
        *reinterpret_cast<uint4 *>(sQ + r * LDK + c) = qv;
    }
    // 2. gates: inclusive scan of g inside the chunk
    if (wave == 0) {
        float gv = 0.f, bv = 0.f;
        if (lane < nv) {
            const int64_t gi = (s * n_tokens + t0 + lane) * n_heads + h;
            gv = g[gi];
            bv = beta[gi];
        }
        float x = gv;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const float glast = __shfl(x, nv - 1, 64);
        const bool ok = lane < nv;
        sG[lane] = x;
        sG[C + lane] = ok ? bv : 0.f;
        sG[2 * C + lane] = ok ? expf(x) : 0.f;
        sG[3 * C + lane] = ok ? expf(glast - x) : 0.f;
        if (lane == 0) sG[4 * C] = expf(glast);
    }
    __syncthreads();

    // 3. K K^T and Q K^T on the 10 lower tiles each (MFMA), decay masks applied
    const int gq = lane >> 4, cl = lane & 15;
    for (int job = wave; job < 20; job += kPrepThreads / 64) {
        const bool isq = job >= 10;
        int tr, tc;
        lower_tile(isq ? job - 10 : job, tr, tc);
        const E *Am = isq ? sQ : sK;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const Frag<BF16> a = lds_frag<BF16>(Am, LDK, 16 * tr + cl, 32 * ks, gq);
            const Frag<BF16> b = lds_frag<BF16>(sK, LDK, 16 * tc + cl, 32 * ks, gq);
            acc = mma(a, b, acc);
        }
        const int col = 16 * tc + cl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * tr + 4 * gq + j;
            const float dec = (col <= row) ? expf(sG[row] - sG[col]) : 0.f;
            if (isq)
                sP[row * LDA + col] = dec * acc[j];
            else
                sA[row * LDA + col] = (col < row) ? sG[C + row] * dec * acc[j] : 0.f;
        }
    }
    __syncthreads();

    // 4. T = (I + A)^{-1}.  (a) 16x16 diagonal blocks: lane = (block, column),
    //    forward substitution down the column.
    if (wave == 0) {
        const int b = lane >> 4, c = lane & 15;
        const float *Ab = sA + (16 * b) * LDA + 16 * b;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) acc = fmaf(-Ab[r * LDA + m], x[m], acc);
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(16 * b + r) * LDA + 16 * b + c] = x[r];
    }
    __syncthreads();
    // (b) off-diagonal blocks, one block diagonal at a time:
    //     X = A[i-rows][16j : 16i] T[16j : 16i][j-cols],  T_ij = -T_ii X
    for (int dd = 1; dd < 4; ++dd) {
        const int nb = 4 - dd;
        for (int e = tid; e < nb * 256; e += kPrepThreads) {
            const int blk = e >> 8, r = (e >> 4) & 15, c = e & 15;
            const int i = blk + dd, j = blk;
            const float *arow = sA + (16 * i + r) * LDA;
            float acc = 0.f;
            for (int u = 16 * j; u < 16 * i; ++u) acc = fmaf(arow[u], sT[u * LDA + 16 * j + c], acc);
            sX[(blk * 16 + r) * 17 + c] = acc;
        }
        __syncthreads();
        for (int e = tid; e < nb * 256; e += kPrepThreads) {
            const int blk = e >> 8, r = (e >> 4) & 15, c = e & 15;
            const int i = blk + dd, j = blk;
            const float *trow = sT + (16 * i + r) * LDA + 16 * i;
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) acc = fmaf(trow[m], sX[(blk * 16 + m) * 17 + c], acc);
            sT[(16 * i + r) * LDA + 16 * j + c] = -acc;
        }
        __syncthreads();
    }

    // 5. T, P (upper triangles written as zeros) and gates to the workspace
    unsigned char *dst = ws + chunk_id * W::kBytes;
    E *wT = reinterpret_cast<E *>(dst + W::kT);
    E *wP = reinterpret_cast<E *>(dst + W::kP);
    for (int i = tid; i < C * C / VE; i += kPrepThreads) {
        const int r = (i * VE) / C, c0 = (i * VE) % C;
        E vt[VE], vp[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const int c = c0 + e;
            vt[e] = from_f<E>(c <= r ? sT[r * LDA + c] : 0.f);
            vp[e] = from_f<E>(c <= r ? sP[r * LDA + c] : 0.f);
        }
        *reinterpret_cast<uint4 *>(wT + i * VE) = *reinterpret_cast<const uint4 *>(vt);
        *reinterpret_cast<uint4 *>(wP + i * VE) = *reinterpret_cast<const uint4 *>(vp);
    }
    float4 *wG = reinterpret_cast<float4 *>(dst + W::kGates);
    if (tid < C) wG[tid] = make_float4(sG[C + tid], sG[2 * C + tid], sG[3 * C + tid], sG[4 * C]);
}

// ---- the chunk-to-chunk scan -----------------------------------------------------

template <int D, int NW, bool BF16>
struct ScanSmem {
    using E = typename Elem<BF16>::T;
    static constexpr int RW = 16 * NW;               // value rows per workgroup
    static constexpr int PAD = BF16 ? 8 : 4;
    static constexpr int LDK = D + PAD;               // sK, sQ rows
    static constexpr int LDT = C + PAD;               // sKt, sT, sP rows
    static constexpr int LDV = RW + PAD;              // sV rows
    static constexpr int kK = 0;
    static constexpr int kQ = kK + C * LDK * sizeof(E);
    static constexpr int kKt = kQ + C * LDK * sizeof(E);
    static constexpr int kT = kKt + D * LDT * sizeof(E);
    static constexpr int kP = kT + C * LDT * sizeof(E);
    static constexpr int kV = kP + C * LDT * sizeof(E);
    static constexpr int kG = kV + C * LDV * sizeof(E);
    static constexpr int kBytes = kG + 4 * C * 4;
    static_assert(kBytes <= 160 * 1024, "LDS budget");
};

// Per-thread staging registers for one chunk (global -> registers -> LDS).
template <int D, int NW, bool BF16>
struct Stage {
    using E = typename Elem<BF16>::T;
    static constexpr int NT = NW * 64;
    static constexpr int VE = 16 / sizeof(E);
    static constexpr int RW = 16 * NW;
    static constexpr int NK = (C * D / VE + NT - 1) / NT;      // K (and Q) vectors
    static constexpr int NTP = (C * C / VE + NT - 1) / NT;     // T (and P) vectors
    static constexpr int NV = (C * RW / VE + NT - 1) / NT;     // V vectors
    static constexpr int NG = (4 * C / 4 + NT - 1) / NT;       // gate float4 vectors
    uint4 k[NK], q[NK], t[NTP], p[NTP], v[NV], gt[NG];
};

template <int D, int NW, bool BF16>
__device__ __forceinline__ void stage_fetch(Stage<D, NW, BF16> &st, const void *q, const void *k,
                                            const void *v, const unsigned char *wsc,
                                            int64_t s, int64_t h, int64_t t0, int nv,
                                            int64_t n_tokens, int64_t n_heads, int v0, int tid)
{
    using S = Stage<D, NW, BF16>;
    using E = typename Elem<BF16>::T;
    using W = WsLayout<BF16>;
    constexpr int VPR = D / S::VE;
#pragma unroll
    for (int i = 0; i < S::NK; ++i) {
        const int idx = tid + i * S::NT;
        st.k[i] = st.q[i] = make_uint4(0, 0, 0, 0);
        if (idx < C * VPR) {
            const int r = idx / VPR, c = (idx - r * VPR) * S::VE;
            if (r < nv) {
                const int64_t off = ((s * n_tokens + t0 + r) * n_heads + h) * D + c;
                st.k[i] = *reinterpret_cast<const uint4 *>(static_cast<const E *>(k) + off);
                st.q[i] = *reinterpret_cast<const uint4 *>(static_cast<const E *>(q) + off);
            }
        }
    }
    const uint4 *wT = reinterpret_cast<const uint4 *>(wsc + W::kT);
    const uint4 *wP = reinterpret_cast<const uint4 *>(wsc + W::kP);
#pragma unroll
    for (int i = 0; i < S::NTP; ++i) {
        const int idx = tid + i * S::NT;
        if (idx < C * C / S::VE) {
            st.t[i] = wT[idx];
            st.p[i] = wP[idx];
        }
    }
    constexpr int VPV = S::RW / S::VE;  // vectors per V row of this workgroup
#pragma unroll
    for (int i = 0; i < S::NV; ++i) {
        const int idx = tid + i * S::NT;
        st.v[i] = make_uint4(0, 0, 0, 0);
        if (idx < C * VPV) {
            const int r = idx / VPV, c = (idx - r * VPV) * S::VE;
            if (r < nv) {
                const int64_t off = ((s * n_tokens + t0 + r) * n_heads + h) * D + v0 + c;
                st.v[i] = *reinterpret_cast<const uint4 *>(static_cast<const E *>(v) + off);
            }
        }
    }
    const uint4 *wG = reinterpret_cast<const uint4 *>(wsc + W::kGates);
#pragma unroll
    for (int i = 0; i < S::NG; ++i) {
        const int idx = tid + i * S::NT;
        if (idx < C) st.gt[i] = wG[idx];
    }
}

template <int D, int NW, bool BF16>
__device__ __forceinline__ void stage_commit(const Stage<D, NW, BF16> &st, unsigned char *smem,
                                             int tid)
{
    using S = Stage<D, NW, BF16>;
    using L = ScanSmem<D, NW, BF16>;
    using E = typename Elem<BF16>::T;
    E *sK = reinterpret_cast<E *>(smem + L::kK);
    E *sQ = reinterpret_cast<E *>(smem + L::kQ);
    E *sKt = reinterpret_cast<E *>(smem + L::kKt);
    E *sT = reinterpret_cast<E *>(smem + L::kT);
    E *sP = reinterpret_cast<E *>(smem + L::kP);
    E *sV = reinterpret_cast<E *>(smem + L::kV);
    float *sG = reinterpret_cast<float *>(smem + L::kG);
    constexpr int VPR = D / S::VE;
#pragma unroll
    for (int i = 0; i < S::NK; ++i) {
        const int idx = tid + i * S::NT;
        if (idx < C * VPR) {
            const int r = idx / VPR, c = (idx - r * VPR) * S::VE;
            *reinterpret_cast<uint4 *>(sK + r * L::LDK + c) = st.k[i];
            *reinterpret_cast<uint4 *>(sQ + r * L::LDK + c) = st.q[i];
            const E *ke = reinterpret_cast<const E *>(&st.k[i]);
#pragma unroll
            for (int e = 0; e < S::VE; ++e) sKt[(c + e) * L::LDT + r] = ke[e];
        }
    }
#pragma unroll
    for (int i = 0; i < S::NTP; ++i) {
        const int idx = tid + i * S::NT;
        if (idx < C * C / S::VE) {
            const int r = (idx * S::VE) / C, c = (idx * S::VE) % C;
            *reinterpret_cast<uint4 *>(sT + r * L::LDT + c) = st.t[i];
            *reinterpret_cast<uint4 *>(sP + r * L::LDT + c) = st.p[i];
        }
    }
    constexpr int VPV = S::RW / S::VE;
#pragma unroll
    for (int i = 0; i < S::NV; ++i) {
        const int idx = tid + i * S::NT;
        if (idx < C * VPV) {
            const int r = idx / VPV, c = (idx - r * VPV) * S::VE;
            *reinterpret_cast<uint4 *>(sV + r * L::LDV + c) = st.v[i];
        }
    }
#pragma unroll
    for (int i = 0; i < S::NG; ++i) {
        const int idx = tid + i * S::NT;
        if (idx < C) *reinterpret_cast<uint4 *>(sG + 4 * idx) = st.gt[i];
    }
}

// Workgroups are numbered so that the row blocks of one (seq, head) share the
// low three bits of the block id: consecutive ids go to different XCDs, so this
// keeps a head's workgroups on one XCD, where its K, Q, T and P hit in L2.
template <int D, int NW, bool BF16>
__global__ __launch_bounds__(NW * 64) void chunk_scan_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *state_in, void *__restrict__ out, float *state_out,
    const unsigned char *__restrict__ ws, int64_t n_tokens, int64_t n_heads, int64_t n_sh,
    int n_chunks, float scale)
{
    using E = typename Elem<BF16>::T;
    using L = ScanSmem<D, NW, BF16>;
    using W = WsLayout<BF16>;
    constexpr int RW = L::RW;
    constexpr int NRB = D / RW;  // row blocks per head
    extern __shared__ __align__(16) unsigned char smem[];
    const E *sK = reinterpret_cast<const E *>(smem + L::kK);
    const E *sQ = reinterpret_cast<const E *>(smem + L::kQ);
    const E *sKt = reinterpret_cast<const E *>(smem + L::kKt);
    const E *sT = reinterpret_cast<const E *>(smem + L::kT);
    const E *sP = reinterpret_cast<const E *>(smem + L::kP);
    const E *sV = reinterpret_cast<const E *>(smem + L::kV);
    const float *sG = reinterpret_cast<const float *>(smem + L::kG);

    const int64_t b = blockIdx.x;
    const int64_t sh = (b / (8 * NRB)) * 8 + (b & 7);
    const int rb = static_cast<int>((b >> 3) % NRB);
    if (sh >= n_sh) return;  // whole workgroup leaves before any barrier
    const int64_t s = sh / n_heads, h = sh - s * n_heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gq = lane >> 4, cl = lane & 15;
    const int v0 = rb * RW;                 // first value row of the workgroup
    const int vrow = v0 + 16 * wave + cl;   // this lane's value row (column of M^T)

    // M^T tiles in accumulator layout: Mt[kt][j] = M[vrow][16 kt + 4 gq + j]
    floatx4 Mt[D / 16];
    const int64_t st_off = sh * D * D + int64_t(vrow) * D;
#pragma unroll
    for (int kt = 0; kt < D / 16; ++kt) {
        if (state_in) {
            const float4 m = *reinterpret_cast<const float4 *>(state_in + st_off + 16 * kt + 4 * gq);
            Mt[kt] = floatx4{m.x, m.y, m.z, m.w};
        } else {
            Mt[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }

    const unsigned char *wsh = ws + sh * n_chunks * W::kBytes;
    Stage<D, NW, BF16> st;
    stage_fetch<D, NW, BF16>(st, q, k, v, wsh, s, h, 0, static_cast<int>(min<int64_t>(C, n_tokens)),
                             n_tokens, n_heads, v0, tid);
    for (int n = 0; n < n_chunks; ++n) {
        const int64_t t0 = int64_t(n) * C;
        const int nv = static_cast<int>(min<int64_t>(C, n_tokens - t0));
        stage_commit<D, NW, BF16>(st, smem, tid);
        __syncthreads();
        if (n + 1 < n_chunks) {
            const int64_t t1 = t0 + C;
            stage_fetch<D, NW, BF16>(st, q, k, v, wsh + (n + 1) * W::kBytes, s, h, t1,
                                     static_cast<int>(min<int64_t>(C, n_tokens - t1)), n_tokens,
                                     n_heads, v0, tid);
        }

        // B operands of M^T, one per 32 keys
        Frag<BF16> bm[D / 32];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) bm[ks] = acc_frag<BF16>(Mt[2 * ks], Mt[2 * ks + 1]);

        // X_K = K M^T, X_Q = Q M^T  (tokens x this wave's 16 value rows)
        floatx4 xk[4], xq[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            xk[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
            xq[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                xk[tt] = mma(lds_frag<BF16>(sK, L::LDK, 16 * tt + cl, 32 * ks, gq), bm[ks], xk[tt]);
                xq[tt] = mma(lds_frag<BF16>(sQ, L::LDK, 16 * tt + cl, 32 * ks, gq), bm[ks], xq[tt]);
            }
        }
        // E = beta (V - e^gam X_K)
        floatx4 e[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * tt + 4 * gq + j;
                const float vv = to_f(sV[t * L::LDV + 16 * wave + cl]);
                e[tt][j] = sG[4 * t] * (vv - sG[4 * t + 1] * xk[tt][j]);
            }
        }
        const Frag<BF16> be0 = acc_frag<BF16>(e[0], e[1]);
        const Frag<BF16> be1 = acc_frag<BF16>(e[2], e[3]);
        // Delta = T E (T lower triangular: token tiles 0-1 need only k block 0)
        floatx4 dl[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            dl[tt] = mma(lds_frag<BF16>(sT, L::LDT, 16 * tt + cl, 0, gq), be0,
                         floatx4{0.f, 0.f, 0.f, 0.f});
            if (tt >= 2) dl[tt] = mma(lds_frag<BF16>(sT, L::LDT, 16 * tt + cl, 32, gq), be1, dl[tt]);
        }
        // O = (e^gam X_Q + P Delta) / sqrt(d)
        const Frag<BF16> bd0 = acc_frag<BF16>(dl[0], dl[1]);
        const Frag<BF16> bd1 = acc_frag<BF16>(dl[2], dl[3]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            floatx4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = sG[4 * (16 * tt + 4 * gq + j) + 1] * xq[tt][j];
            o = mma(lds_frag<BF16>(sP, L::LDT, 16 * tt + cl, 0, gq), bd0, o);
            if (tt >= 2) o = mma(lds_frag<BF16>(sP, L::LDT, 16 * tt + cl, 32, gq), bd1, o);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * tt + 4 * gq + j;
                if (t < nv) {
                    const int64_t off = ((s * n_tokens + t0 + t) * n_heads + h) * D + vrow;
                    static_cast<E *>(out)[off] = from_f<E>(scale * o[j]);
                }
            }
        }
        // M^T <- e^{gam_last} M^T + K^T diag(e^{gam_last - gam}) Delta
        floatx4 ds[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j) ds[tt][j] = sG[4 * (16 * tt + 4 * gq + j) + 2] * dl[tt][j];
        const Frag<BF16> bs0 = acc_frag<BF16>(ds[0], ds[1]);
        const Frag<BF16> bs1 = acc_frag<BF16>(ds[2], ds[3]);
        const float eC = sG[3];
#pragma unroll
        for (int kt = 0; kt < D / 16; ++kt) {
            floatx4 m = Mt[kt] * eC;
            m = mma(lds_frag<BF16>(sKt, L::LDT, 16 * kt + cl, 0, gq), bs0, m);
            m = mma(lds_frag<BF16>(sKt, L::LDT, 16 * kt + cl, 32, gq), bs1, m);
            Mt[kt] = m;
        }
        __syncthreads();
    }

#pragma unroll
    for (int kt = 0; kt < D / 16; ++kt)
        *reinterpret_cast<float4 *>(state_out + st_off + 16 * kt + 4 * gq) =
            make_float4(Mt[kt][0], Mt[kt][1], Mt[kt][2], Mt[kt][3]);
}

template <int D, bool BF16>
hipError_t launch_prep(const Problem &p, unsigned char *ws, int n_chunks, hipStream_t stream)
{
    using L = PrepSmem<D, BF16>;
    auto kern = chunk_prep_kernel<D, BF16>;
    static bool attr_set = false;  // one-time attribute; same value every time
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::kBytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int64_t blocks = p.n_seqs * p.n_heads * n_chunks;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(kPrepThreads), L::kBytes,
                       stream, p.q, p.k, p.g, p.beta, ws, p.n_tokens, p.n_heads, n_chunks);
    return hipGetLastError();
}

template <int D, int NW, bool BF16>
hipError_t launch_scan(const Problem &p, const unsigned char *ws, int n_chunks, hipStream_t stream)
{
    using L = ScanSmem<D, NW, BF16>;
    auto kern = chunk_scan_kernel<D, NW, BF16>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::kBytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    constexpr int NRB = D / (16 * NW);
    const int64_t n_sh = p.n_seqs * p.n_heads;
    const int64_t blocks = (n_sh + 7) / 8 * 8 * NRB;
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(NW * 64), L::kBytes, stream,
                       p.q, p.k, p.v, p.state_in, p.out, p.state_out, ws, p.n_tokens, p.n_heads,
                       n_sh, n_chunks, scale);
    return hipGetLastError();
}

// Waves per scan workgroup: as many as still leave at least 256 workgroups
// (one per compute unit), at least one.
template <int D, bool BF16>
hipError_t launch_chunk_d(const Problem &p, unsigned char *ws, hipStream_t stream)
{
    const int n_chunks = static_cast<int>((p.n_tokens + C - 1) / C);
    hipError_t e = launch_prep<D, BF16>(p, ws, n_chunks, stream);
    if (e != hipSuccess) return e;
    const int64_t n_sh = p.n_seqs * p.n_heads;
    if constexpr (D % 64 == 0) {
        if (n_sh * (D / 64) >= 256) return launch_scan<D, 4, BF16>(p, ws, n_chunks, stream);
    }
    if (n_sh * (D / 32) >= 256) return launch_scan<D, 2, BF16>(p, ws, n_chunks, stream);
    return launch_scan<D, 1, BF16>(p, ws, n_chunks, stream);
}

template <bool BF16>
hipError_t launch_chunk_t(const Problem &p, unsigned char *ws, hipStream_t stream)
{
    switch (p.head_dim) {
    case 32: return launch_chunk_d<32, BF16>(p, ws, stream);
    case 64: return launch_chunk_d<64, BF16>(p, ws, stream);
    case 96: return launch_chunk_d<96, BF16>(p, ws, stream);
    case 128: return launch_chunk_d<128, BF16>(p, ws, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t chunk_workspace_bytes(int bf16, int64_t n_seqs, int64_t n_tokens, int64_t n_heads, int)
{
    const int64_t n_chunks = (n_tokens + C - 1) / C;
    const int64_t per = bf16 ? WsLayout<true>::kBytes : WsLayout<false>::kBytes;
    return static_cast<size_t>(n_seqs * n_heads * n_chunks * per);
}

hipError_t launch_chunked(const Problem &p, void *workspace, hipStream_t stream)
{
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    return p.bf16 ? launch_chunk_t<true>(p, ws, stream) : launch_chunk_t<false>(p, ws, stream);
}

}  // namespace gdn
