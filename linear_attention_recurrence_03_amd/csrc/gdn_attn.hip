// gdn_attn.hip -- decode flash attention for gfx950 (MI355X): a few queries
// (n_q < 20) against a key/value cache, the "vector" case of the "ggml attention
// kernels" model card (section "flash_attn").
//
// Per sequence s, query head h (key/value head j = h / (n_heads / n_heads_kv):
// grouped-query attention read in place, no expanded copy) and query i:
//     score_t = scale (q_i . k_t) + f16(mask[s][i][t])        t < n_kv
//     out_i   = sum_t softmax(score)_t v_t
// The card's kernel casts the additive mask to f16 and accumulates in f16; here the
// mask is rounded to f16 the same way and everything else runs in fp32.  A row with
// no finite score (fully masked, or an empty cache) gives zeros.
//
// Work split (memory-bound: every key/value byte is read once per row group):
//   attn_split_kernel   one workgroup per (seq, key/value head, group of up to four
//                       (query head, query) rows, range of cache tokens).  Per tile of
//                       64 tokens: four threads score one token against the rows
//                       (a quarter of its key row each, 16-byte loads all issued
//                       before the products), one wave per row updates the running
//                       max / sum and turns scores into weights, then the waves
//                       accumulate weights x value rows with lanes owning 8
//                       consecutive columns (whole value rows per load instruction,
//                       a wave's loads of the tile in flight together).  The partial (max, sum, weighted values) of the
//                       token range goes to the workspace, or straight to the output
//                       when the cache is not split.
//   attn_combine_kernel merges the token ranges of each row.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 attn_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float attn_floatx4 __attribute__((ext_vector_type(4)));

constexpr int kAttnThreads = 256;  // four waves
constexpr int kAttnTile = 64;      // cache tokens per tile (four threads each when scoring)
constexpr int kAttnRows = 4;       // (query head, query) rows per workgroup
constexpr int kAttnSplitUnit = 64; // token ranges are multiples of this
constexpr int kAttnTargetBlocks = 2048;  // workgroups to aim for (about 8 per CU)

template <bool BF16>
struct AttnElem;
template <>
struct AttnElem<true> {
    using T = uint16_t;
};
template <>
struct AttnElem<false> {
    using T = float;
};

// eight consecutive elements as fp32
template <bool BF16>
__device__ __forceinline__ void load8(const typename AttnElem<BF16>::T *p, float (&x)[8])
{
    if constexpr (BF16) {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

__device__ __forceinline__ float mask_f16(float m)
{
    return __half2float(__float2half_rn(m));
}

// exp(a - b) with the conventions of the online softmax: b = -inf means nothing seen
// (weight 0); a = b = -inf keeps a running sum unchanged.
__device__ __forceinline__ float exp_diff(float a, float b)
{
    if (a == b) return 1.f;
    return (a == -INFINITY) ? 0.f : __expf(a - b);
}

struct AttnArgs {
    const void *q, *k, *v;
    const float *mask;          // (S, 1, n_q, n_kv) or null
    void *out;                  // (S, n_q, H, D)
    float *part;                // per (row, split): D weighted sums, max, sum
    float scale;
    int64_t n_heads, n_heads_kv, n_q, n_kv;
    int groups;                 // row groups per (seq, key/value head)
    int n_split, split_len;     // token ranges per row and their length
};

template <int D, bool BF16>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(AttnArgs a)
{
    using E = typename AttnElem<BF16>::T;
    constexpr int QW = D / 4;            // key elements per scoring thread
    constexpr int LPR = D / 8;           // lanes covering one value row
    constexpr int SPW = 64 / LPR;        // value rows per wave instruction
    constexpr int STREAMS = 4 * SPW;     // partial accumulators per column
    constexpr int TPW = kAttnTile / 4;   // tile tokens per wave in the value pass
    static_assert(D % 64 == 0 && D <= 256, "head width");
    static_assert(kAttnTile == 64 && TPW % SPW == 0, "tile");

    __shared__ __align__(16) float sQ[kAttnRows][D];
    __shared__ float sS[kAttnRows][kAttnTile];
    __shared__ float sCorr[kAttnRows];
    __shared__ __align__(16) float sAcc[STREAMS][kAttnRows][D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const int split = static_cast<int>(b % a.n_split);
    const int64_t u = b / a.n_split;
    const int grp = static_cast<int>(u % a.groups);
    const int64_t sj = u / a.groups;                  // s * n_heads_kv + j
    const int64_t s = sj / a.n_heads_kv, j = sj - s * a.n_heads_kv;
    const int64_t hg = a.n_heads / a.n_heads_kv;      // query heads per key/value head
    const int64_t rows_here = hg * a.n_q;

    // row r of this group: query head j*hg + R / n_q, query R % n_q
    int64_t rh[kAttnRows], ri[kAttnRows];
    bool rv[kAttnRows];
#pragma unroll
    for (int r = 0; r < kAttnRows; ++r) {
        const int64_t R = int64_t(grp) * kAttnRows + r;
        rv[r] = R < rows_here;
        rh[r] = rv[r] ? j * hg + R / a.n_q : 0;
        ri[r] = rv[r] ? R % a.n_q : 0;
    }

    // scaled query rows (zeros for unused rows)
    for (int x = tid; x < kAttnRows * D; x += kAttnThreads) {
        const int r = x / D, c = x - r * D;
        float val = 0.f;
        if (rv[r]) {
            const int64_t off = ((s * a.n_heads + rh[r]) * a.n_q + ri[r]) * D + c;
            if constexpr (BF16)
                val = bf16_to_f32(static_cast<const uint16_t *>(a.q)[off]);
            else
                val = static_cast<const float *>(a.q)[off];
        }
        sQ[r][c] = val * a.scale;
    }

    // bf16: the query rows as the A operand of the scoring product (row m = lane % 16
    // of the group, dimensions 32 ks + 8 (lane / 16) .. +7; rows past the group's
    // four, or unused, are zero); the scale is applied to the fp32 scores
    uint4 aq[D / 32];
    if constexpr (BF16) {
        const int m = lane & 15, g = lane >> 4;
        const int64_t R = int64_t(grp) * kAttnRows + m;
        const bool ok = m < kAttnRows && R < rows_here;
        const int64_t off = ok ? ((s * a.n_heads + j * hg + R / a.n_q) * a.n_q + R % a.n_q) * D : 0;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            aq[ks] = ok ? *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + off +
                                                           32 * ks + 8 * g)
                        : make_uint4(0u, 0u, 0u, 0u);
    }

    const int64_t t_begin = int64_t(split) * a.split_len;
    const int64_t t_end = t_begin + a.split_len < a.n_kv ? t_begin + a.split_len : a.n_kv;
    const E *kbase = static_cast<const E *>(a.k) + (s * a.n_heads_kv + j) * a.n_kv * D;
    const E *vbase = static_cast<const E *>(a.v) + (s * a.n_heads_kv + j) * a.n_kv * D;

    float m_run = -INFINITY, l_run = 0.f;   // wave r's row statistics (row r = wave)
    const int stream = wave * SPW + lane / LPR, col = (lane % LPR) * 8;
    const int tok = tid >> 2, qtr = tid & 3;  // scoring: four threads per token
    float acc[kAttnRows][8];
#pragma unroll
    for (int r = 0; r < kAttnRows; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
    __syncthreads();

    for (int64_t t0 = t_begin; t0 < t_end; t0 += kAttnTile) {
        const int last = static_cast<int>(t_end - t0 < kAttnTile ? t_end - t0 : kAttnTile) - 1;
        // the value rows of the tile do not depend on the scores: their loads go out
        // with the key loads, so a tile costs one memory round trip.  Wave w takes
        // tile tokens TPW w .. TPW w + TPW - 1; tokens past the end read the last
        // valid row and get weight 0.
        const int tl0 = TPW * wave + lane / LPR;
        uint4 vraw[TPW / SPW][BF16 ? 1 : 2];
#pragma unroll
        for (int it = 0; it < TPW / SPW; ++it) {
            const int tl = tl0 + it * SPW;
            const uint4 *src = reinterpret_cast<const uint4 *>(
                vbase + (t0 + (tl < last ? tl : last)) * D + col);
#pragma unroll
            for (int h = 0; h < (BF16 ? 1 : 2); ++h) vraw[it][h] = src[h];
        }
        // 1. scores.  bf16: wave w scores tile tokens 16 w .. 16 w + 15 against the
        //    group's rows on MFMA (A: the query rows, B: lane (g, n) holds key row
        //    16 w + n, dimensions 32 ks + 8 g .. +7); lane n of the first 16 holds the
        //    four rows' scores of token 16 w + n.  fp32: thread (tok, qtr) takes a
        //    quarter of key row t0 + tok.  Rows past the end read the last valid one
        //    and are masked below; all loads are issued before the first product.
        if constexpr (BF16) {
            const int n = lane & 15, g = lane >> 4, tokl = 16 * wave + n;
            const E *kr = kbase + (t0 + (tokl < last ? tokl : last)) * D + 8 * g;
            uint4 bk[D / 32];
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) bk[ks] = *reinterpret_cast<const uint4 *>(kr + 32 * ks);
            attn_floatx4 sc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                sc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(attn_bf16x8_t, aq[ks]),
                                                              __builtin_bit_cast(attn_bf16x8_t, bk[ks]),
                                                              sc4, 0, 0, 0);
            if (g == 0) {
                const int64_t t = t0 + tokl;
#pragma unroll
                for (int r = 0; r < kAttnRows; ++r) {
                    float v = sc4[r] * a.scale;
                    if (!rv[r] || tokl > last)
                        v = -INFINITY;
                    else if (a.mask)
                        v += mask_f16(a.mask[(s * a.n_q + ri[r]) * a.n_kv + t]);
                    sS[r][tokl] = v;
                }
            }
        } else {
            const E *kr = kbase + (t0 + (tok < last ? tok : last)) * D + qtr * QW;
            constexpr int KU = BF16 ? 1 : 2;          // 16-byte units per 8 elements
            uint4 kraw[QW / 8][KU];
#pragma unroll
            for (int c = 0; c < QW / 8; ++c)
#pragma unroll
                for (int h = 0; h < KU; ++h) kraw[c][h] = reinterpret_cast<const uint4 *>(kr + 8 * c)[h];
            float sc[kAttnRows];
#pragma unroll
            for (int r = 0; r < kAttnRows; ++r) sc[r] = 0.f;
#pragma unroll
            for (int c = 0; c < QW / 8; ++c) {
                float x8[8];
                load8<BF16>(reinterpret_cast<const E *>(&kraw[c][0]), x8);
#pragma unroll
                for (int r = 0; r < kAttnRows; ++r) {
                    const float4 q0 = *reinterpret_cast<const float4 *>(&sQ[r][qtr * QW + 8 * c]);
                    const float4 q1 = *reinterpret_cast<const float4 *>(&sQ[r][qtr * QW + 8 * c + 4]);
                    sc[r] = fmaf(q0.x, x8[0], fmaf(q0.y, x8[1], fmaf(q0.z, x8[2], fmaf(q0.w, x8[3], sc[r]))));
                    sc[r] = fmaf(q1.x, x8[4], fmaf(q1.y, x8[5], fmaf(q1.z, x8[6], fmaf(q1.w, x8[7], sc[r]))));
                }
            }
#pragma unroll
            for (int r = 0; r < kAttnRows; ++r) {
                sc[r] += __shfl_xor(sc[r], 1, 64);
                sc[r] += __shfl_xor(sc[r], 2, 64);
            }
            if (qtr == 0) {
                const int64_t t = t0 + tok;
#pragma unroll
                for (int r = 0; r < kAttnRows; ++r) {
                    float v = sc[r];
                    if (!rv[r] || tok > last)
                        v = -INFINITY;
                    else if (a.mask)
                        v += mask_f16(a.mask[(s * a.n_q + ri[r]) * a.n_kv + t]);
                    sS[r][tok] = v;
                }
            }
        }
        __syncthreads();

        // 2. wave r: running max and sum of row r; scores become weights
        {
            const int r = wave;
            const float x = sS[r][lane];
            float mt = x;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o, 64));
            const float m_new = fmaxf(m_run, mt);
            const float corr = exp_diff(m_run, m_new);
            const float p = (x == -INFINITY) ? 0.f : __expf(x - m_new);
            sS[r][lane] = p;
            float ps = p;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) ps += __shfl_xor(ps, o, 64);
            l_run = l_run * corr + ps;
            m_run = m_new;
            if (lane == 0) sCorr[r] = corr;
        }
        __syncthreads();

        // 3. weighted value rows (loaded above)
        {
#pragma unroll
            for (int r = 0; r < kAttnRows; ++r) {
                const float cr = sCorr[r];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] *= cr;
            }
#pragma unroll
            for (int it = 0; it < TPW / SPW; ++it) {
                const int tl = tl0 + it * SPW;
                float vx[8];
                load8<BF16>(reinterpret_cast<const E *>(&vraw[it][0]), vx);
#pragma unroll
                for (int r = 0; r < kAttnRows; ++r) {
                    const float p = sS[r][tl];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(p, vx[e], acc[r][e]);
                }
            }
        }
        __syncthreads();
    }

    // 4. merge the streams of each column; wave r holds row r's max and sum
#pragma unroll
    for (int r = 0; r < kAttnRows; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) sAcc[stream][r][col + e] = acc[r][e];
    if (lane == 0) {
        sS[wave][0] = m_run;
        sS[wave][1] = l_run;
    }
    __syncthreads();
    for (int x = tid; x < kAttnRows * D; x += kAttnThreads) {
        const int r = x / D, c = x - r * D;
        if (!rv[r]) continue;
        float sum = 0.f;
#pragma unroll
        for (int st = 0; st < STREAMS; ++st) sum += sAcc[st][r][c];
        const float m = sS[r][0], l = sS[r][1];
        const int64_t row = (s * a.n_q + ri[r]) * a.n_heads + rh[r];   // (s, i, h)
        if (a.n_split == 1) {
            const float o = (l > 0.f) ? sum / l : 0.f;
            if constexpr (BF16)
                static_cast<uint16_t *>(a.out)[row * D + c] = f32_to_bf16(o);
            else
                static_cast<float *>(a.out)[row * D + c] = o;
        } else {
            float *pp = a.part + (row * a.n_split + split) * (D + 2);
            pp[c] = sum;
            if (c == 0) {
                pp[D] = m;
                pp[D + 1] = l;
            }
        }
    }
}

// One wave per (seq, query, head) row: merges its token ranges.  Lanes load the
// ranges' maxima and sums in parallel (64 ranges per pass), then each lane adds the
// weighted partial sums of its D/64 columns with the weights taken from the lanes
// that hold them.
template <int D, bool BF16>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a)
{
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x;
    const int ns = a.n_split;
    const float *pp = a.part + row * ns * (D + 2);
    float M = -INFINITY;
    for (int i0 = 0; i0 < ns; i0 += 64)
        if (i0 + lane < ns) M = fmaxf(M, pp[(i0 + lane) * (D + 2) + D]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float den = 0.f, num[D / 64];
#pragma unroll
    for (int e = 0; e < D / 64; ++e) num[e] = 0.f;
    for (int i0 = 0; i0 < ns; i0 += 64) {
        float w = 0.f;
        if (i0 + lane < ns) {
            const float *pi = pp + (i0 + lane) * (D + 2);
            const float m = pi[D];
            w = (m == -INFINITY) ? 0.f : __expf(m - M);
            den = fmaf(w, pi[D + 1], den);
        }
        const int cnt = ns - i0 < 64 ? ns - i0 : 64;
        for (int i = 0; i < cnt; i += 8) {
            float x[8][D / 64], wi[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int ii = i + q < cnt ? i + q : cnt - 1;
                wi[q] = __shfl(w, ii, 64);
                if (i + q >= cnt) wi[q] = 0.f;
#pragma unroll
                for (int e = 0; e < D / 64; ++e) x[q][e] = pp[(i0 + ii) * (D + 2) + lane + 64 * e];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int e = 0; e < D / 64; ++e) num[e] = fmaf(wi[q], x[q][e], num[e]);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o, 64);
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
        const float o = (den > 0.f) ? num[e] / den : 0.f;
        const int64_t idx = row * D + lane + 64 * e;
        if constexpr (BF16)
            static_cast<uint16_t *>(a.out)[idx] = f32_to_bf16(o);
        else
            static_cast<float *>(a.out)[idx] = o;
    }
}

template <int D, bool BF16>
hipError_t launch_attn_d(const AttnProblem &p, void *ws, hipStream_t stream)
{
    AttnArgs a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.mask = p.mask;
    a.out = p.out;
    a.part = static_cast<float *>(ws);
    a.scale = p.scale;
    a.n_heads = p.n_heads;
    a.n_heads_kv = p.n_heads_kv;
    a.n_q = p.n_q;
    a.n_kv = p.n_kv;
    const AttnSplit sp = attn_split(p.n_seqs, p.n_heads, p.n_heads_kv, p.n_q, p.n_kv);
    a.groups = sp.groups;
    a.n_split = sp.n_split;
    a.split_len = sp.split_len;
    const int64_t blocks = p.n_seqs * p.n_heads_kv * sp.groups * int64_t(sp.n_split);
    const int64_t rows = p.n_seqs * p.n_q * p.n_heads;
    if (!grid_fits(blocks, kAttnThreads) || !grid_fits(rows, 64)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_split_kernel<D, BF16>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kAttnThreads), 0, stream, a);
    if (sp.n_split > 1) {
        hipLaunchKernelGGL((attn_combine_kernel<D, BF16>), dim3(static_cast<uint32_t>(rows)),
                           dim3(64), 0, stream, a);
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_attn_t(const AttnProblem &p, void *ws, hipStream_t stream)
{
    switch (p.head_dim) {
    case 64: return launch_attn_d<64, BF16>(p, ws, stream);
    case 128: return launch_attn_d<128, BF16>(p, ws, stream);
    case 256: return launch_attn_d<256, BF16>(p, ws, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

namespace {

struct SplitSizes {
    int64_t groups, n_split, split_len;
};

SplitSizes split_sizes(int64_t n_seqs, int64_t n_heads, int64_t n_heads_kv, int64_t n_q,
                       int64_t n_kv)
{
    SplitSizes sp;
    const int64_t hg = n_heads / n_heads_kv;
    sp.groups = (hg * n_q + kAttnRows - 1) / kAttnRows;
    const int64_t units = n_seqs * n_heads_kv * sp.groups;
    const int64_t max_split = (n_kv + kAttnSplitUnit - 1) / kAttnSplitUnit;
    int64_t ns = (kAttnTargetBlocks + units - 1) / units;
    if (ns > max_split) ns = max_split;
    if (ns < 1) ns = 1;
    // equal ranges, each a multiple of the unit
    int64_t len = (n_kv + ns - 1) / ns;
    len = (len + kAttnSplitUnit - 1) / kAttnSplitUnit * kAttnSplitUnit;
    if (len < kAttnSplitUnit) len = kAttnSplitUnit;
    ns = (n_kv + len - 1) / len;
    if (ns < 1) ns = 1;
    sp.n_split = ns;
    sp.split_len = len;
    return sp;
}

}  // namespace

AttnSplit attn_split(int64_t n_seqs, int64_t n_heads, int64_t n_heads_kv, int64_t n_q,
                     int64_t n_kv)
{
    const SplitSizes z = split_sizes(n_seqs, n_heads, n_heads_kv, n_q, n_kv);
    AttnSplit sp;
    sp.groups = static_cast<int>(z.groups);
    sp.n_split = static_cast<int>(z.n_split);
    sp.split_len = static_cast<int>(z.split_len);
    return sp;
}

bool attn_grid_fits(int64_t n_seqs, int64_t n_heads, int64_t n_heads_kv, int64_t n_q,
                    int64_t n_kv)
{
    const SplitSizes z = split_sizes(n_seqs, n_heads, n_heads_kv, n_q, n_kv);
    if (z.groups > INT32_MAX || z.n_split > INT32_MAX || z.split_len > INT32_MAX) return false;
    const int64_t units = n_seqs * n_heads_kv * z.groups;
    return grid_fits(units, kAttnThreads) && units <= INT64_MAX / z.n_split &&
           grid_fits(units * z.n_split, kAttnThreads) && grid_fits(n_seqs * n_q * n_heads, 64);
}

size_t attn_workspace_bytes(int64_t n_seqs, int64_t n_heads, int64_t n_heads_kv, int64_t n_q,
                            int64_t n_kv, int head_dim)
{
    const AttnSplit sp = attn_split(n_seqs, n_heads, n_heads_kv, n_q, n_kv);
    if (sp.n_split <= 1) return 0;
    return static_cast<size_t>(n_seqs * n_q * n_heads * sp.n_split * (head_dim + 2)) *
           sizeof(float);
}

hipError_t launch_attn(const AttnProblem &p, void *workspace, hipStream_t stream)
{
    return p.bf16 ? launch_attn_t<true>(p, workspace, stream)
                  : launch_attn_t<false>(p, workspace, stream);
}

}  // namespace gdn
