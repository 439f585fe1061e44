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
//                         16x16x4 fp32 for fp32 inputs), with the chunk's K, Q, T,
//                         P and V staged in LDS (K^T operands come from
//                         transposing LDS reads); the next chunk's loads
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
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, bf16x2_t));
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

typedef short short4_t __attribute__((ext_vector_type(4)));

// A operand whose rows are the key channels of a token-major LDS matrix: lane
// (g, i) gets base[t0 + k(g, j)][key0 + i] for the eight j, i.e. eight tokens of
// one key.  For bf16 this is two ds_read_b64_tr_b16: inside each group of 16
// lanes, lane i receives element j = (i mod 4)-th 16-bit value fetched by lane
// 4j + i/4, so lane p of group g fetches row t0 + 4g + p/4 (then 16 rows lower),
// keys key0 + 4 (p mod 4) .. +3.
template <bool BF16>
__device__ __forceinline__ Frag<BF16> lds_frag_tr(const typename Elem<BF16>::T *base, int ld,
                                                  int t0, int key0, int lane)
{
    Frag<BF16> f;
    const int g = lane >> 4, p = lane & 15;
    if constexpr (BF16) {
        const uint16_t *a1 = base + (t0 + 4 * g + (p >> 2)) * ld + key0 + 4 * (p & 3);
        const uint16_t *a2 = a1 + 16 * ld;
        typedef __attribute__((address_space(3))) short4_t lds_short4;
        const short4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(a1));
        const short4_t r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(a2));
        const uint2 u1 = __builtin_bit_cast(uint2, r1);
        const uint2 u2 = __builtin_bit_cast(uint2, r2);
        f.u = make_uint4(u1.x, u1.y, u2.x, u2.y);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f.v[j] = base[(t0 + 4 * g + j) * ld + key0 + p];
            f.v[4 + j] = base[(t0 + 16 + 4 * g + j) * ld + key0 + p];
        }
    }
    return f;
}

// B operand from two stacked accumulator tiles (rows 0-15 and 16-31 of the k range).
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

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global load and store of the wave, which would stall on the next
// chunk's prefetch and on output stores that nothing in the workgroup reads.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- workspace layout, per (seq, head, chunk) ----------------------------------
//   T     [C][C] elements   (fp32 or bf16, like q/k/v)
//   P     [C][C] elements
//   gates [4][C] fp32: beta_r, e^{gam_r}, e^{gam_last - gam_r}, then e^{gam_last}
//                      repeated C times
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
    static constexpr int kG = kT + C * LDA * 4;
    static constexpr int kBytes = kG + (4 * C + 4) * 4;
};

// Lower 16x16 tiles (tr >= tc) of a 4x4 tile grid, in a fixed order.
__device__ __forceinline__ void lower_tile(int ix, int &tr, int &tc)
{
    tr = (ix >= 6) ? 3 : (ix >= 3) ? 2 : (ix >= 1) ? 1 : 0;
    tc = ix - tr * (tr + 1) / 2;
}

// Upper 16x16 tiles (tr < tc), fixed order.
__device__ __forceinline__ void upper_tile(int ix, int &tr, int &tc)
{
    tr = (ix >= 5) ? 2 : (ix >= 3) ? 1 : 0;
    tc = tr + 1 + (ix - (tr == 0 ? 0 : tr == 1 ? 3 : 5));
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
    float *sG = reinterpret_cast<float *>(smem + L::kG);  // gam, beta, e^gam, e^{last-gam}, e^last

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t chunk_id = blockIdx.x;
    const int64_t sh = chunk_id / n_chunks;
    const int n = static_cast<int>(chunk_id - sh * n_chunks);
    const int64_t s = sh / n_heads, h = sh - s * n_heads;
    const int64_t t0 = int64_t(n) * C;
    const int nv = static_cast<int>(min<int64_t>(C, n_tokens - t0));
    unsigned char *dst = ws + chunk_id * W::kBytes;
    E *wT = reinterpret_cast<E *>(dst + W::kT);
    E *wP = reinterpret_cast<E *>(dst + W::kP);

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
    lds_barrier();

    const int gq = lane >> 4, cl = lane & 15;
    // 3. A = beta e^{gam_r - gam_s} K K^T (strictly lower), on the 10 lower tiles
    for (int job = wave; job < 10; job += kPrepThreads / 64) {
        int tr, tc;
        lower_tile(job, tr, tc);
        Frag<BF16> fa[D / 32], fb[D / 32];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            fa[ks] = lds_frag<BF16>(sK, LDK, 16 * tr + cl, 32 * ks, gq);
            fb[ks] = lds_frag<BF16>(sK, LDK, 16 * tc + cl, 32 * ks, gq);
        }
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) acc = mma(fa[ks], fb[ks], acc);
        const int col = 16 * tc + cl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * tr + 4 * gq + j;
            sA[row * LDA + col] =
                (col < row) ? sG[C + row] * __expf(sG[row] - sG[col]) * acc[j] : 0.f;
        }
    }
    lds_barrier();

    if (wave == 0) {
        // 4a. 16x16 diagonal blocks of T = (I + A)^{-1}: lane = (block, column),
        //     forward substitution down the column.
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
    } else {
        // 3b (other waves, meanwhile). P = e^{gam_r - gam_s} Q K^T (lower incl.
        //    diagonal), written straight from the accumulators; upper tiles zero.
        for (int job = wave - 1; job < 16; job += kPrepThreads / 64 - 1) {
            int tr, tc;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            if (job < 10) {
                lower_tile(job, tr, tc);
                Frag<BF16> fa[D / 32], fb[D / 32];
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    fa[ks] = lds_frag<BF16>(sQ, LDK, 16 * tr + cl, 32 * ks, gq);
                    fb[ks] = lds_frag<BF16>(sK, LDK, 16 * tc + cl, 32 * ks, gq);
                }
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) acc = mma(fa[ks], fb[ks], acc);
            } else {
                upper_tile(job - 10, tr, tc);
            }
            const int col = 16 * tc + cl;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * tr + 4 * gq + j;
                const float pv = (col <= row) ? __expf(sG[row] - sG[col]) * acc[j] : 0.f;
                wP[row * C + col] = from_f<E>(pv);
            }
        }
    }
    lds_barrier();

    // 4b. off-diagonal blocks of T, one block diagonal at a time, on fp32 MFMA:
    //     X = A[i rows][16j : 16i] T[16j : 16i][j cols] (inner length 16 (i-j)),
    //     T_ij = -T_ii X.  X stays in accumulator registers: for the second
    //     product, k step jj pairs lane group g with row 4g + jj of X.
    for (int dd = 1; dd < 4; ++dd) {
        if (wave < 4 - dd) {
            const int j = wave, i = wave + dd;
            floatx4 X = {0.f, 0.f, 0.f, 0.f};
            for (int st = 0; st < 4 * dd; ++st) {
                const int u = 16 * j + 4 * st + gq;
                X = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * i + cl) * LDA + u],
                                                         sT[u * LDA + 16 * j + cl], X, 0, 0, 0);
            }
            floatx4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                Y = __builtin_amdgcn_mfma_f32_16x16x4f32(
                    sT[(16 * i + cl) * LDA + 16 * i + 4 * gq + jj], X[jj], Y, 0, 0, 0);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sT[(16 * i + 4 * gq + jj) * LDA + 16 * j + cl] = -Y[jj];
        }
        lds_barrier();
    }

    // 5. T (upper triangle as zeros) and gates to the workspace
    for (int i = tid; i < C * C / VE; i += kPrepThreads) {
        const int r = (i * VE) / C, c0 = (i * VE) % C;
        E vt[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const int c = c0 + e;
            vt[e] = from_f<E>(c <= r ? sT[r * LDA + c] : 0.f);
        }
        *reinterpret_cast<uint4 *>(wT + i * VE) = *reinterpret_cast<const uint4 *>(vt);
    }
    float *wG = reinterpret_cast<float *>(dst + W::kGates);
    if (tid < C) {
        wG[tid] = sG[C + tid];
        wG[C + tid] = sG[2 * C + tid];
        wG[2 * C + tid] = sG[3 * C + tid];
        wG[3 * C + tid] = sG[4 * C];
    }
}

// ---- the chunk-to-chunk scan -----------------------------------------------------
//
// One workgroup = four waves for RW = 16 VT value rows of one (seq, head):
//   wave 0  "chain": carries those rows of M^T in registers and per chunk does
//           X = K M^T, E = beta (V - e^gam X), Delta = T E and the state update --
//           the serial dependency from chunk to chunk;
//   wave 1  "output": while the chain wave works on X, E and Delta it forms
//           e^gam Q M^T from the M^T fragments the chain wave published, then
//           after a mid-step barrier adds P Delta and stores O;
//   waves 2, 3  "producers": issue the next chunk's loads (K, Q, T, P, V,
//           gates) global -> LDS with global_load_lds (16 bytes per lane) into
//           the stage not in use, and wait for them; a compute unit ingests
//           these loads faster when more than one wave issues them.
// Each wave sits on its own SIMD.  K, Q, T and P are read from LDS once per
// workgroup per chunk; LDS rows are padded by 16 bytes so that fragment reads
// spread over the banks.  Rows past the end of a partial chunk are loaded from
// the last valid row: the prep kernel gives them beta = e^gam = 0, so they
// contribute nothing, and finite data keeps 0 * x = 0.

constexpr int kScanThreads = 256;

template <int D, bool BF16, int VT>
struct ScanCfg {
    using E = typename Elem<BF16>::T;
    static constexpr int RW = 16 * VT;               // value rows per workgroup
    static constexpr int kStages = BF16 ? 2 : 1;
    static constexpr int ES = sizeof(E);
    static constexpr int RK = D * ES + 16;          // sK, sQ row stride (bytes)
    static constexpr int RT = C * ES + 16;          // sT, sP row stride
    static constexpr int RV = RW * ES + 16;         // sV row stride
    static constexpr int kK = 0;
    static constexpr int kQ = kK + C * RK;
    static constexpr int kT = kQ + C * RK;
    static constexpr int kP = kT + C * RT;
    static constexpr int kV = kP + C * RT;
    static constexpr int kG = kV + C * RV;
    static constexpr int kStage = (kG + 4 * C * 4 + 1023) / 1024 * 1024;
    static constexpr int KS = D / 32;
    static constexpr int kFrags = (KS + 2) * VT;    // M^T and Delta fragments
    static constexpr int kPub = kStages * kStage;
    static constexpr int kBytes = kPub + 64 * kFrags * int(sizeof(Frag<BF16>));
    static_assert(kBytes <= 160 * 1024, "LDS budget");
    // 1 KiB LDS-DMA blocks per region (64 padded rows are a whole number of blocks)
    static constexpr int NBK = C * RK / 1024;
    static constexpr int NBT = C * RT / 1024;
    static constexpr int NBV = C * RV / 1024;
    static_assert(C * RK % 1024 == 0 && C * RT % 1024 == 0 && C * RV % 1024 == 0, "blocks");
};

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

// One 16-byte-per-lane LDS-DMA: lane l's 16 bytes (from base + off) land at
// lds + 16 l.  base is wave-uniform; off is a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16(const unsigned char *base, uint32_t off, void *lds)
{
    __builtin_amdgcn_global_load_lds((global_cvoid *)(base + off), (lds_void *)(lds), 16, 0, 0);
}

// Wait for this wave's outstanding global loads (LDS-DMA included).
__device__ __forceinline__ void wait_vmem()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unconstrained
}

// Byte offset, inside one chunk's data, of the 16 bytes lane `lane` loads for LDS
// block `blk` of a padded region: rows of `rowb` valid bytes stored with stride
// `stride`; pad slots read row 0.  `gstride` is the source row stride; rows past
// nv read row nv - 1.
__device__ __forceinline__ uint32_t dma_src_offset(int blk, int lane, int rowb, int stride,
                                                   uint32_t gstride, int nv)
{
    const int o = blk * 1024 + lane * 16;
    const int r = o / stride, b = o - r * stride;
    const uint32_t v = uint32_t(min(r, nv - 1)) * gstride + uint32_t(b);
    return b < rowb ? v : 0u;
}

struct ScanPtrs {
    const unsigned char *k, *q, *v;   // token 0 of this (seq, head); v at the first value row
    const unsigned char *ws;          // this (seq, head)'s chunk 0 in the workspace
    int64_t hd_bytes;                 // token stride in bytes (64 of them fit in 32 bits)
};

// Producer waves: issue the LDS-DMA loads of chunk n into stage buffer `buf`;
// producer `part` of 2 takes every other 1 KiB block.
template <int D, bool BF16, int VT>
__device__ __forceinline__ void scan_issue(const ScanPtrs &pt, unsigned char *buf, int n, int nv,
                                           int part, int lane)
{
    using F = ScanCfg<D, BF16, VT>;
    using W = WsLayout<BF16>;
    const int64_t tb = int64_t(n) * C * pt.hd_bytes;
    const uint32_t hdb = static_cast<uint32_t>(pt.hd_bytes);
    const unsigned char *kb = pt.k + tb, *qb = pt.q + tb, *vb = pt.v + tb;
    const unsigned char *wsc = pt.ws + int64_t(n) * W::kBytes;
    // K on producer 0, Q on producer 1 (same lane offsets); T/P/V blocks alternate
#pragma unroll
    for (int blk = 0; blk < F::NBK; ++blk) {
        const uint32_t off = dma_src_offset(blk, lane, D * F::ES, F::RK, hdb, nv);
        dma16(part == 0 ? kb : qb, off, buf + (part == 0 ? F::kK : F::kQ) + 1024 * blk);
    }
#pragma unroll
    for (int blk = 0; blk < F::NBT; ++blk) {
        const uint32_t off = dma_src_offset(blk, lane, C * F::ES, F::RT, C * F::ES, C);
        dma16(wsc + (part == 0 ? W::kT : W::kP), off, buf + (part == 0 ? F::kT : F::kP) + 1024 * blk);
    }
#pragma unroll
    for (int blk = 0; blk < F::NBV; ++blk)
        if ((blk & 1) == part)
            dma16(vb, dma_src_offset(blk, lane, F::RW * F::ES, F::RV, hdb, nv), buf + F::kV + 1024 * blk);
    if (part == (F::NBV & 1)) dma16(wsc + W::kGates, 16u * lane, buf + F::kG);
}

// Fragment loaders on the padded LDS layout.  A operand row `row`, k elements
// k0 + {4g..4g+3} and k0 + 16 + {4g..4g+3}.
template <bool BF16>
__device__ __forceinline__ Frag<BF16> frag_rows(const unsigned char *base, int stride, int row,
                                                int k0, int g)
{
    Frag<BF16> f;
    constexpr int ES = BF16 ? 2 : 4;
    const unsigned char *p = base + row * stride + (k0 + 4 * g) * ES;
    if constexpr (BF16) {
        const uint2 lo = *reinterpret_cast<const uint2 *>(p);
        const uint2 hi = *reinterpret_cast<const uint2 *>(p + 32);
        f.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
        const float4 lo = *reinterpret_cast<const float4 *>(p);
        const float4 hi = *reinterpret_cast<const float4 *>(p + 64);
        f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
        f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
    }
    return f;
}

// Operand whose rows are columns c0 + (lane mod 16) of a row-major LDS matrix and
// whose k values are rows t0 + {4g..4g+3}, t0 + 16 + {4g..4g+3} (eight rows of
// one column).  bf16: two ds_read_b64_tr_b16 (see lds_frag_tr).
template <bool BF16>
__device__ __forceinline__ Frag<BF16> frag_cols(const unsigned char *base, int stride, int t0,
                                                int c0, int lane)
{
    Frag<BF16> f;
    const int g = lane >> 4, p = lane & 15;
    if constexpr (BF16) {
        const unsigned char *a1 = base + (t0 + 4 * g + (p >> 2)) * stride + (c0 + 4 * (p & 3)) * 2;
        typedef __attribute__((address_space(3))) short4_t lds_short4;
        const short4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(a1));
        const short4_t r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(a1 + 16 * stride));
        const uint2 u1 = __builtin_bit_cast(uint2, r1);
        const uint2 u2 = __builtin_bit_cast(uint2, r2);
        f.u = make_uint4(u1.x, u1.y, u2.x, u2.y);
    } else {
        const float *col = reinterpret_cast<const float *>(base + (c0 + p) * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f.v[j] = *reinterpret_cast<const float *>(reinterpret_cast<const unsigned char *>(col) +
                                                      (t0 + 4 * g + j) * stride);
            f.v[4 + j] = *reinterpret_cast<const float *>(reinterpret_cast<const unsigned char *>(col) +
                                                          (t0 + 16 + 4 * g + j) * stride);
        }
    }
    return f;
}

// Values of one LDS column at four consecutive rows t..t+3 (accumulator layout
// rows 4g+j of a tile): lane (g, i) gets base[t0 + 4g + j][c0 + i], j = 0..3.
template <bool BF16>
__device__ __forceinline__ floatx4 col4(const unsigned char *base, int stride, int t0, int c0,
                                        int lane)
{
    const int g = lane >> 4, p = lane & 15;
    floatx4 r;
    if constexpr (BF16) {
        // one transposing read: lane 4j + i/4 fetches row t0 + 4g + j, columns
        // c0 + 4 (i/4) .. +3; lane i receives column c0 + i of the four rows
        const unsigned char *a = base + (t0 + 4 * g + (p >> 2)) * stride + (c0 + 4 * (p & 3)) * 2;
        typedef __attribute__((address_space(3))) short4_t lds_short4;
        const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(a));
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = bf16_to_f32(static_cast<uint16_t>(v[j]));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = *reinterpret_cast<const float *>(base + (t0 + 4 * g + j) * stride + (c0 + p) * 4);
    }
    return r;
}

// Chain wave, one chunk.  All LDS reads of the step (K rows, T, gates, V and the
// transposed K for the update) are issued first; then X = K M^T, E = beta (V -
// e^gam X), Delta = T E (published, then barrier B for the output wave) and the
// state update M^T <- e^{gam_last} M^T + K^T diag(e^{gam_last - gam}) Delta,
// whose new fragments are published for the next step.
template <int D, bool BF16, int VT>
__device__ __forceinline__ void chain_step(floatx4 (&Mt)[VT][D / 16], const unsigned char *buf,
                                           Frag<BF16> *pub, int lane)
{
    using F = ScanCfg<D, BF16, VT>;
    constexpr int KS = F::KS;
    const int gq = lane >> 4, cl = lane & 15;
    const float *sG = reinterpret_cast<const float *>(buf + F::kG);
    Frag<BF16> ak[4][KS];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ak[tt][ks] = frag_rows<BF16>(buf + F::kK, F::RK, 16 * tt + cl, 32 * ks, gq);
    Frag<BF16> at[6];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        at[tt] = frag_rows<BF16>(buf + F::kT, F::RT, 16 * tt + cl, 0, gq);
        if (tt >= 2) at[2 + tt] = frag_rows<BF16>(buf + F::kT, F::RT, 16 * tt + cl, 32, gq);
    }
    floatx4 bt[4], eg[4], edec[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int t = 16 * tt + 4 * gq;
        const float4 b4 = *reinterpret_cast<const float4 *>(sG + t);
        const float4 e4 = *reinterpret_cast<const float4 *>(sG + C + t);
        const float4 d4 = *reinterpret_cast<const float4 *>(sG + 2 * C + t);
        bt[tt] = floatx4{b4.x, b4.y, b4.z, b4.w};
        eg[tt] = floatx4{e4.x, e4.y, e4.z, e4.w};
        edec[tt] = floatx4{d4.x, d4.y, d4.z, d4.w};
    }
    const float eC = sG[3 * C];
    floatx4 vv[VT][4];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) vv[vt][tt] = col4<BF16>(buf + F::kV, F::RV, 16 * tt, 16 * vt, lane);
    Frag<BF16> akt[D / 16][2];
#pragma unroll
    for (int kt = 0; kt < D / 16; ++kt) {
        akt[kt][0] = frag_cols<BF16>(buf + F::kK, F::RK, 0, 16 * kt, lane);
        akt[kt][1] = frag_cols<BF16>(buf + F::kK, F::RK, 32, 16 * kt, lane);
    }

    floatx4 dl[VT][4];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
        Frag<BF16> bm[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bm[ks] = acc_frag<BF16>(Mt[vt][2 * ks], Mt[vt][2 * ks + 1]);
        floatx4 xk[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) xk[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) xk[tt] = mma(ak[tt][ks], bm[ks], xk[tt]);
        floatx4 e[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j) e[tt][j] = bt[tt][j] * fmaf(-eg[tt][j], xk[tt][j], vv[vt][tt][j]);
        const Frag<BF16> be0 = acc_frag<BF16>(e[0], e[1]);
        const Frag<BF16> be1 = acc_frag<BF16>(e[2], e[3]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) dl[vt][tt] = mma(at[tt], be0, floatx4{0.f, 0.f, 0.f, 0.f});
        dl[vt][2] = mma(at[4], be1, dl[vt][2]);
        dl[vt][3] = mma(at[5], be1, dl[vt][3]);
        pub[(VT * KS + 2 * vt) * 64 + lane] = acc_frag<BF16>(dl[vt][0], dl[vt][1]);
        pub[(VT * KS + 2 * vt + 1) * 64 + lane] = acc_frag<BF16>(dl[vt][2], dl[vt][3]);
    }
    lds_barrier();  // B: Delta_n is published
    Frag<BF16> bs[VT][2];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
        floatx4 ds[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) ds[tt] = edec[tt] * dl[vt][tt];
        bs[vt][0] = acc_frag<BF16>(ds[0], ds[1]);
        bs[vt][1] = acc_frag<BF16>(ds[2], ds[3]);
    }
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int kt = 0; kt < D / 16; ++kt) Mt[vt][kt] = mma(akt[kt][0], bs[vt][0], Mt[vt][kt] * eC);
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int kt = 0; kt < D / 16; ++kt) Mt[vt][kt] = mma(akt[kt][1], bs[vt][1], Mt[vt][kt]);
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            pub[(vt * KS + ks) * 64 + lane] = acc_frag<BF16>(Mt[vt][2 * ks], Mt[vt][2 * ks + 1]);
}

// Output wave, one chunk: reads Q, P and gates, forms e^gam Q M^T from the
// published M^T fragments, waits at barrier B for Delta, adds P Delta and stores
// O / sqrt(d) for valid tokens.  orow points at out[(s, first token of the chunk,
// h, first value row + lane%16)].
template <int D, bool BF16, int VT>
__device__ __forceinline__ void output_step(const unsigned char *buf, const Frag<BF16> *pub,
                                            int lane, typename Elem<BF16>::T *orow, int64_t hd,
                                            int nv, float scale)
{
    using F = ScanCfg<D, BF16, VT>;
    using E = typename Elem<BF16>::T;
    constexpr int KS = F::KS;
    const int gq = lane >> 4, cl = lane & 15;
    const float *sG = reinterpret_cast<const float *>(buf + F::kG);
    Frag<BF16> aq[4][KS];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            aq[tt][ks] = frag_rows<BF16>(buf + F::kQ, F::RK, 16 * tt + cl, 32 * ks, gq);
    Frag<BF16> ap[6];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        ap[tt] = frag_rows<BF16>(buf + F::kP, F::RT, 16 * tt + cl, 0, gq);
        if (tt >= 2) ap[2 + tt] = frag_rows<BF16>(buf + F::kP, F::RT, 16 * tt + cl, 32, gq);
    }
    floatx4 eg[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const float4 e4 = *reinterpret_cast<const float4 *>(sG + C + 16 * tt + 4 * gq);
        eg[tt] = floatx4{e4.x, e4.y, e4.z, e4.w};
    }
    floatx4 o[VT][4];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
        Frag<BF16> bm[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bm[ks] = pub[(vt * KS + ks) * 64 + lane];
        floatx4 xq[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) xq[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) xq[tt] = mma(aq[tt][ks], bm[ks], xq[tt]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) o[vt][tt] = eg[tt] * xq[tt];
    }
    lds_barrier();  // B: Delta_n is published
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
        const Frag<BF16> bd0 = pub[(VT * KS + 2 * vt) * 64 + lane];
        const Frag<BF16> bd1 = pub[(VT * KS + 2 * vt + 1) * 64 + lane];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) o[vt][tt] = mma(ap[tt], bd0, o[vt][tt]);
        o[vt][2] = mma(ap[4], bd1, o[vt][2]);
        o[vt][3] = mma(ap[5], bd1, o[vt][3]);
        E *ov = orow + 16 * vt;
        if (nv == C) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[(16 * tt + 4 * gq + j) * hd] = from_f<E>(scale * o[vt][tt][j]);
        } else {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 16 * tt + 4 * gq + j;
                    if (t < nv) ov[t * hd] = from_f<E>(scale * o[vt][tt][j]);
                }
        }
    }
}

// Workgroups are numbered so that the row blocks of one (seq, head) share the
// low three bits of the block id: consecutive ids go to different XCDs, so this
// keeps a head's workgroups on one XCD, where its K, Q, T and P hit in L2.
template <int D, bool BF16, int VT>
__global__ __launch_bounds__(kScanThreads) void chunk_scan_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *state_in, void *__restrict__ out, float *state_out,
    const unsigned char *__restrict__ ws, int64_t n_tokens, int64_t n_heads, int64_t n_sh,
    int n_chunks, float scale)
{
    using F = ScanCfg<D, BF16, VT>;
    using E = typename Elem<BF16>::T;
    using W = WsLayout<BF16>;
    constexpr int NRB = D / F::RW;  // row blocks per head
    constexpr int S = F::kStages;
    extern __shared__ __align__(16) unsigned char smem[];

    const int64_t b = blockIdx.x;
    const int64_t sh = (b / (8 * NRB)) * 8 + (b & 7);
    const int rb = static_cast<int>((b >> 3) % NRB);
    if (sh >= n_sh) return;  // whole workgroup leaves before any barrier
    const int64_t s = sh / n_heads, h = sh - s * n_heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int v0 = rb * F::RW;                       // first value row of the workgroup
    const int64_t hd = n_heads * D;
    const int64_t tok0 = (s * n_tokens * n_heads + h) * D;
    ScanPtrs pt;
    pt.k = static_cast<const unsigned char *>(k) + tok0 * F::ES;
    pt.q = static_cast<const unsigned char *>(q) + tok0 * F::ES;
    pt.v = static_cast<const unsigned char *>(v) + (tok0 + v0) * F::ES;
    pt.ws = ws + sh * n_chunks * W::kBytes;
    pt.hd_bytes = hd * F::ES;
    Frag<BF16> *pub = reinterpret_cast<Frag<BF16> *>(smem + F::kPub);
    auto nv_of = [&](int n) { return static_cast<int>(min<int64_t>(C, n_tokens - int64_t(n) * C)); };

    if (wave >= 2) {
        // producers
        const int part = wave - 2;
        if constexpr (S == 2) scan_issue<D, BF16, VT>(pt, smem, 0, nv_of(0), part, lane);
        for (int n = 0; n < n_chunks; ++n) {
            if constexpr (S == 1) scan_issue<D, BF16, VT>(pt, smem, n, nv_of(n), part, lane);
            wait_vmem();
            lds_barrier();  // A: chunk n is in LDS
            if constexpr (S == 2) {
                if (n + 1 < n_chunks)
                    scan_issue<D, BF16, VT>(pt, smem + ((n + 1) & 1) * F::kStage, n + 1,
                                            nv_of(n + 1), part, lane);
            }
            lds_barrier();  // B
            if constexpr (S == 1) lds_barrier();
        }
        return;
    }

    // M^T tiles in accumulator layout: Mt[vt][kt][j] = M[v0 + 16 vt + lane%16][16 kt + 4 g + j]
    const int64_t st_off = sh * D * D + int64_t(v0 + (lane & 15)) * D + 4 * (lane >> 4);
    if (wave == 0) {
        floatx4 Mt[VT][D / 16];
#pragma unroll
        for (int vt = 0; vt < VT; ++vt)
#pragma unroll
            for (int kt = 0; kt < D / 16; ++kt) {
                if (state_in) {
                    const float4 m = *reinterpret_cast<const float4 *>(state_in + st_off +
                                                                       16 * vt * D + 16 * kt);
                    Mt[vt][kt] = floatx4{m.x, m.y, m.z, m.w};
                } else {
                    Mt[vt][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
        for (int vt = 0; vt < VT; ++vt)
#pragma unroll
            for (int ks = 0; ks < F::KS; ++ks)
                pub[(vt * F::KS + ks) * 64 + lane] = acc_frag<BF16>(Mt[vt][2 * ks], Mt[vt][2 * ks + 1]);
        for (int n = 0; n < n_chunks; ++n) {
            const unsigned char *buf = smem + (S == 2 ? (n & 1) : 0) * F::kStage;
            lds_barrier();  // A: chunk n is in LDS; M^T_n is published
            chain_step<D, BF16, VT>(Mt, buf, pub, lane);  // contains barrier B
            if constexpr (S == 1) lds_barrier();
        }
#pragma unroll
        for (int vt = 0; vt < VT; ++vt)
#pragma unroll
            for (int kt = 0; kt < D / 16; ++kt)
                *reinterpret_cast<float4 *>(state_out + st_off + 16 * vt * D + 16 * kt) =
                    make_float4(Mt[vt][kt][0], Mt[vt][kt][1], Mt[vt][kt][2], Mt[vt][kt][3]);
    } else {
        E *orow = static_cast<E *>(out) + tok0 + v0 + (lane & 15);
        for (int n = 0; n < n_chunks; ++n) {
            const unsigned char *buf = smem + (S == 2 ? (n & 1) : 0) * F::kStage;
            lds_barrier();  // A
            output_step<D, BF16, VT>(buf, pub, lane, orow + int64_t(n) * C * hd, hd, nv_of(n),
                                     scale);  // contains barrier B
            if constexpr (S == 1) lds_barrier();
        }
    }
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

template <int D, bool BF16, int VT>
hipError_t launch_scan(const Problem &p, const unsigned char *ws, int n_chunks, hipStream_t stream)
{
    using F = ScanCfg<D, BF16, VT>;
    auto kern = chunk_scan_kernel<D, BF16, VT>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, F::kBytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    constexpr int NRB = D / F::RW;
    const int64_t n_sh = p.n_seqs * p.n_heads;
    const int64_t blocks = (n_sh + 7) / 8 * 8 * NRB;
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(kScanThreads), F::kBytes,
                       stream, p.q, p.k, p.v, p.state_in, p.out, p.state_out, ws, p.n_tokens,
                       p.n_heads, n_sh, n_chunks, scale);
    return hipGetLastError();
}

// Scan workgroups hold 16 value rows each while that still leaves at most one
// workgroup per compute unit (few heads: more parallel chains), else 32.
template <int D, bool BF16>
hipError_t launch_chunk_d(const Problem &p, unsigned char *ws, hipStream_t stream)
{
    const int n_chunks = static_cast<int>((p.n_tokens + C - 1) / C);
    hipError_t e = launch_prep<D, BF16>(p, ws, n_chunks, stream);
    if (e != hipSuccess) return e;
    const int64_t n_sh = p.n_seqs * p.n_heads;
    if (n_sh * (D / 16) <= 256) return launch_scan<D, BF16, 1>(p, ws, n_chunks, stream);
    return launch_scan<D, BF16, 2>(p, ws, n_chunks, stream);
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
