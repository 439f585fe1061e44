// gdn_attn.hip -- decode flash attention for gfx950 (MI355X): a few queries
// (n_q < 20) against a key/value cache, the "vector" case of the "ggml attention
// kernels" model card (section "flash_attn").
//
// Per sequence s, query head h (key/value head j = h / (n_heads / n_heads_kv):
// grouped-query attention read in place, no expanded copy) and query i:
//     score_t = scale (q_i . k_t) + f16(mask[s][i][t])        t < n_kv
//     out_i   = sum_t softmax(score)_t v_t
// The card's kernel casts the additive mask to f16 and accumulates in f16; here the
// mask is rounded to f16 the same way and everything else runs in fp32, except
// that the bf16 kernel multiplies bf16 operands on MFMA (the query and key rows as
// given, and the softmax weights rounded to bf16 for the weighted sum of value
// rows), accumulating in fp32.  A row with no finite score (fully masked, or an
// empty cache) gives zeros.
//
// Work split (memory-bound: every key/value byte is read once per row group): one
// workgroup per (seq, key/value head, group of up to four (query head, query) rows,
// range of cache tokens), ranges sized for about 1,024 workgroups.  Per tile of 64
// tokens, one wave per row updates the running max / sum and turns scores into
// weights; the products differ by type:
//   attn_split_mma_kernel  (bf16) each wave scores its 16 tokens on MFMA and owns a
//                          quarter of the output columns, accumulating V^T P^T on
//                          MFMA from the tile's value rows staged in LDS by LDS-DMA
//                          (read back with transposing reads); the next tile's key
//                          rows are loaded while the current tile is reduced;
//   attn_split_kernel      (fp32) four threads score one token (a quarter of its key
//                          row each), and the waves accumulate weights x value rows
//                          with lanes owning 8 consecutive columns, merged at the end.
// The partial (max, sum, weighted values) of each token range goes to the
// workspace, or straight to the output when the cache is not split;
// attn_combine_kernel merges the token ranges of each row.
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
constexpr int kAttnTargetBlocks = 1024;  // workgroups to aim for: one round of the bf16 kernel (4 per CU)

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

// The kernels take these as separate arguments in this order (a struct passed by
// value is not preloaded): the first 14 dwords are what a workgroup's first loads
// need, and this file is built to have the hardware preload them into scalar
// registers at wave launch.  Counts are 32-bit (the rows, the grids and the cache
// length are bounded below 2^31).
struct AttnArgs {
    const void *q, *k, *v;
    uint32_t n_split, groups;   // token ranges per row; row groups per (seq, kv head)
    uint32_t n_heads_kv, hg;    // key/value heads; query heads per key/value head
    uint32_t n_q, n_kv;
    uint32_t split_len;         // tokens per range
    float scale;
    const float *mask;          // (S, 1, n_q, n_kv) or null
    void *out;                  // (S, n_q, H, D)
    float *part;                // per (row, split): D weighted sums, max, sum
};
#define ATTN_ARGS(a)                                                                          \
    (a).q, (a).k, (a).v, (a).n_split, (a).groups, (a).n_heads_kv, (a).hg, (a).n_q, (a).n_kv, \
        (a).split_len, (a).scale, (a).mask, (a).out, (a).part

template <int D, bool BF16>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(
    const void *q_, const void *k_, const void *v_, uint32_t n_split_, uint32_t groups_,
    uint32_t n_heads_kv_, uint32_t hg_, uint32_t n_q_, uint32_t n_kv_, uint32_t split_len_,
    float scale_, const float *mask_, void *out_, float *part_)
{
    const AttnArgs a{q_, k_, v_, n_split_, groups_, n_heads_kv_, hg_, n_q_, n_kv_, split_len_,
                     scale_, mask_, out_, part_};
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
    // block -> (seq, key/value head, row group, token range), in 32 bits
    const uint32_t b = blockIdx.x;
    const int split = static_cast<int>(b % a.n_split);
    const uint32_t u = b / a.n_split;
    const int grp = static_cast<int>(u % a.groups);
    const uint32_t sj = u / a.groups;                 // s * n_heads_kv + j
    const uint32_t s32 = sj / a.n_heads_kv;
    const int64_t s = s32, j = sj - s32 * a.n_heads_kv;
    const int64_t n_heads = int64_t(a.hg) * a.n_heads_kv;
    const int64_t hg = a.hg;                          // query heads per key/value head
    const int64_t rows_here = hg * a.n_q;

    // row r of this group: query head j*hg + R / n_q, query R % n_q
    int64_t rh[kAttnRows], ri[kAttnRows];
    bool rv[kAttnRows];
#pragma unroll
    for (int r = 0; r < kAttnRows; ++r) {
        const int64_t R = int64_t(grp) * kAttnRows + r;
        rv[r] = R < rows_here;
        rh[r] = rv[r] ? j * hg + uint32_t(R) / a.n_q : 0;
        ri[r] = rv[r] ? uint32_t(R) % a.n_q : 0;
    }

    // scaled query rows (zeros for unused rows)
    for (int x = tid; x < kAttnRows * D; x += kAttnThreads) {
        const int r = x / D, c = x - r * D;
        float val = 0.f;
        if (rv[r]) {
            const int64_t off = ((s * n_heads + rh[r]) * a.n_q + ri[r]) * D + c;
            if constexpr (BF16)
                val = bf16_to_f32(static_cast<const uint16_t *>(a.q)[off]);
            else
                val = static_cast<const float *>(a.q)[off];
        }
        sQ[r][c] = val * a.scale;
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
        // 1. scores: thread (tok, qtr) takes a quarter of key row t0 + tok (rows past
        //    the end read the last valid one and are masked below); all its loads are
        //    issued before the first product
        {
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
        const int64_t row = (s * a.n_q + ri[r]) * n_heads + rh[r];   // (s, i, h)
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

// bf16 decode attention with both products on MFMA.  Same work split as
// attn_split_kernel; per tile of 64 cache tokens:
//   1. each wave loads the key rows of its 16 tokens into registers and issues the
//      LDS-DMA of its share of the tile's value rows (rows padded to 2 (mod 4)
//      16-byte units, which keeps the transposing reads below free of bank
//      conflicts); scores on MFMA as in attn_split_kernel;
//   2. wave r: running max and sum of row r; scores become weights (fp32);
//   3. O^T += V^T P^T on MFMA: wave w owns D/4 output columns; the A operand (V^T:
//      rows = columns of V, k = tokens) comes from transposing LDS reads of the
//      staged tile, the B operand (P^T) from the weights rounded to bf16, zero for
//      rows past the group's four.  Each lane's accumulator holds one row, so the
//      running correction factor is one multiply per lane.
// A wave's output columns are its own: no merge between waves.
template <int D>
struct AttnMmaCfg {
    static constexpr int RS = D * 2 + 32;            // staged value row stride (bytes)
    static constexpr int NB = kAttnTile * RS / 1024; // LDS-DMA blocks per tile
    static constexpr int CW = D / 4;                 // output columns per wave
    static constexpr int MT = CW / 16;               // their 16-column MFMA tiles
    static_assert((RS / 16) % 4 == 2 && kAttnTile * RS % 1024 == 0 && CW % 16 == 0, "layout");
};

// A operand whose rows are columns c0 + (lane mod 16) of the staged tile and whose k
// values are tokens t0 + {4g .. 4g+3}, t0 + 16 + {4g .. 4g+3} (g = lane / 16): two
// ds_read_b64_tr_b16, inside each group of 16 lanes lane p fetching token
// t0 + 4g + p/4 (then 16 tokens later), columns c0 + 4 (p mod 4) .. +3.
__device__ __forceinline__ uint4 attn_vt_frag(const unsigned char *base, int stride, int t0, int c0,
                                              int lane)
{
    typedef short short4v __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) short4v lds_short4v;
    const int g = lane >> 4, p = lane & 15;
    const unsigned char *a1 = base + (t0 + 4 * g + (p >> 2)) * stride + (c0 + 4 * (p & 3)) * 2;
    const short4v r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(a1));
    const short4v r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(a1 + 16 * stride));
    const uint2 u1 = __builtin_bit_cast(uint2, r1), u2 = __builtin_bit_cast(uint2, r2);
    return make_uint4(u1.x, u1.y, u2.x, u2.y);
}

__device__ __forceinline__ uint32_t attn_pack_bf16(float a, float b)
{
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    typedef float float2v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{a, b}, bf16x2v));
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_split_mma_kernel(
    const void *q_, const void *k_, const void *v_, uint32_t n_split_, uint32_t groups_,
    uint32_t n_heads_kv_, uint32_t hg_, uint32_t n_q_, uint32_t n_kv_, uint32_t split_len_,
    float scale_, const float *mask_, void *out_, float *part_)
{
    const AttnArgs a{q_, k_, v_, n_split_, groups_, n_heads_kv_, hg_, n_q_, n_kv_, split_len_,
                     scale_, mask_, out_, part_};
    using F = AttnMmaCfg<D>;
    __shared__ __align__(16) unsigned char sV[kAttnTile * F::RS];
    __shared__ __align__(16) float sS[kAttnRows][kAttnTile];
    __shared__ float sCorr[kAttnRows];
    __shared__ float sML[kAttnRows][2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    // block -> (seq, key/value head, row group, token range), in 32 bits
    const uint32_t b = blockIdx.x;
    const int split = static_cast<int>(b % a.n_split);
    const uint32_t u = b / a.n_split;
    const int grp = static_cast<int>(u % a.groups);
    const uint32_t sj = u / a.groups;                 // s * n_heads_kv + j
    const uint32_t s32 = sj / a.n_heads_kv;
    const int64_t s = s32, j = sj - s32 * a.n_heads_kv;
    const int64_t n_heads = int64_t(a.hg) * a.n_heads_kv;
    const int64_t hg = a.hg;
    const int64_t rows_here = hg * a.n_q;

    bool rv[kAttnRows];
    int64_t ri[kAttnRows];
#pragma unroll
    for (int r = 0; r < kAttnRows; ++r) {
        const int64_t R = int64_t(grp) * kAttnRows + r;
        rv[r] = R < rows_here;
        ri[r] = rv[r] ? uint32_t(R) % a.n_q : 0;
    }

    // query rows as the A operand of the scores (lane row n of the group)
    uint4 aq[D / 32];
    {
        const int64_t R = int64_t(grp) * kAttnRows + n;
        const bool ok = n < kAttnRows && R < rows_here;
        const int64_t off =
            ok ? ((s * n_heads + j * hg + uint32_t(R) / a.n_q) * a.n_q + uint32_t(R) % a.n_q) * D : 0;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            aq[ks] = ok ? *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + off +
                                                           32 * ks + 8 * g)
                        : make_uint4(0u, 0u, 0u, 0u);
    }

    const int64_t t_begin = int64_t(split) * a.split_len;
    const int64_t t_end = t_begin + a.split_len < a.n_kv ? t_begin + a.split_len : a.n_kv;
    const uint16_t *kbase = static_cast<const uint16_t *>(a.k) + (s * a.n_heads_kv + j) * a.n_kv * D;
    const unsigned char *vbase = reinterpret_cast<const unsigned char *>(
        static_cast<const uint16_t *>(a.v) + (s * a.n_heads_kv + j) * a.n_kv * D);

    float m_run = -INFINITY, l_run = 0.f;   // wave r's row statistics (row r = wave)
    attn_floatx4 acc[F::MT];
#pragma unroll
    for (int mt = 0; mt < F::MT; ++mt) acc[mt] = attn_floatx4{0.f, 0.f, 0.f, 0.f};

    // key rows of this wave's 16 tokens of the tile at tt (B operand of the scores);
    // tokens past the end read the last valid row
    const int tokl = 16 * wave + n;
    uint4 bk[D / 32];
    auto load_k = [&](int64_t tt, uint4 (&dstk)[D / 32]) {
        const int lst = static_cast<int>(t_end - tt < kAttnTile ? t_end - tt : kAttnTile) - 1;
        const uint16_t *kr = kbase + (tt + (tokl < lst ? tokl : lst)) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) dstk[ks] = *reinterpret_cast<const uint4 *>(kr + 32 * ks);
    };
    if (t_begin < t_end) load_k(t_begin, bk);
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kAttnTile) {
        const int last = static_cast<int>(t_end - t0 < kAttnTile ? t_end - t0 : kAttnTile) - 1;
        // 1. value rows' LDS-DMA; the key rows of this wave's tokens were loaded
        //    one tile ahead; tokens past the end read the last valid row and get weight 0
        const unsigned char *vt = vbase + t0 * (D * 2);
        for (int i = wave; i < F::NB; i += kAttnThreads / 64)
            dma16(vt, dma_src_offset(i, lane, D * 2, F::RS, D * 2, last + 1), sV + 1024 * i);
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
        const bool more = t0 + kAttnTile < t_end;
        uint4 bkn[D / 32];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) bkn[ks] = bk[ks];
        if (more) {
            load_k(t0 + kAttnTile, bkn);
            wait_vmem_le<D / 32>();  // the value rows have landed; the next keys may not
        } else {
            wait_vmem_le<0>();
        }
        __syncthreads();

        // 2. wave r: running max and sum of row r; scores become weights
        {
            const int r = wave;
            const float x = sS[r][lane];
            float mx = x;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            const float m_new = fmaxf(m_run, mx);
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

        // 3. O^T += V^T P^T for this wave's columns
        {
            const float cr = n < kAttnRows ? sCorr[n < kAttnRows ? n : 0] : 0.f;
#pragma unroll
            for (int mt = 0; mt < F::MT; ++mt) acc[mt] *= cr;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint4 pb = make_uint4(0u, 0u, 0u, 0u);
                if (n < kAttnRows) {
                    const float4 p0 = *reinterpret_cast<const float4 *>(&sS[n][32 * kk + 4 * g]);
                    const float4 p1 = *reinterpret_cast<const float4 *>(&sS[n][32 * kk + 16 + 4 * g]);
                    pb = make_uint4(attn_pack_bf16(p0.x, p0.y), attn_pack_bf16(p0.z, p0.w),
                                    attn_pack_bf16(p1.x, p1.y), attn_pack_bf16(p1.z, p1.w));
                }
#pragma unroll
                for (int mt = 0; mt < F::MT; ++mt) {
                    const uint4 va = attn_vt_frag(sV, F::RS, 32 * kk, wave * F::CW + 16 * mt, lane);
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(attn_bf16x8_t, va), __builtin_bit_cast(attn_bf16x8_t, pb),
                        acc[mt], 0, 0, 0);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) bk[ks] = bkn[ks];
    }

    // 4. lane (g, n < 4) holds row n's columns wave * CW + 16 mt + 4 g .. +3
    if (lane == 0) {
        sML[wave][0] = m_run;
        sML[wave][1] = l_run;
    }
    __syncthreads();
    if (n < kAttnRows) {
        bool ok = false;
        int64_t row = 0;
#pragma unroll
        for (int r = 0; r < kAttnRows; ++r)
            if (r == n) {
                ok = rv[r];
                row = (s * a.n_q + ri[r]) * n_heads + j * hg + uint32_t(grp * kAttnRows + r) / a.n_q;
            }
        if (ok) {
            const float m = sML[n][0], l = sML[n][1];
#pragma unroll
            for (int mt = 0; mt < F::MT; ++mt) {
                const int c = wave * F::CW + 16 * mt + 4 * g;
                if (a.n_split == 1) {
                    const float inv = l > 0.f ? 1.f / l : 0.f;
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + row * D + c) =
                        make_uint2(attn_pack_bf16(acc[mt][0] * inv, acc[mt][1] * inv),
                                   attn_pack_bf16(acc[mt][2] * inv, acc[mt][3] * inv));
                } else {
                    float *pp = a.part + (row * a.n_split + split) * (D + 2);   // 8-byte aligned
                    *reinterpret_cast<float2 *>(pp + c) = make_float2(acc[mt][0], acc[mt][1]);
                    *reinterpret_cast<float2 *>(pp + c + 2) = make_float2(acc[mt][2], acc[mt][3]);
                    if (c == 0) {
                        pp[D] = m;
                        pp[D + 1] = l;
                    }
                }
            }
        }
    }
}

// One wave per (seq, query, head) row: merges its token ranges.  Lanes load the
// ranges' maxima and sums in parallel (64 ranges per pass), then each lane adds the
// weighted partial sums of its D/64 columns with the weights taken from the lanes
// that hold them.
template <int D, bool BF16>
__global__ __launch_bounds__(64) void attn_combine_kernel(const float *part, void *out,
                                                          uint32_t n_split)
{
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x;
    const int ns = n_split;
    const float *pp = part + row * ns * (D + 2);
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
            static_cast<uint16_t *>(out)[idx] = f32_to_bf16(o);
        else
            static_cast<float *>(out)[idx] = o;
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
    a.n_heads_kv = static_cast<uint32_t>(p.n_heads_kv);
    a.hg = static_cast<uint32_t>(p.n_heads / p.n_heads_kv);
    a.n_q = static_cast<uint32_t>(p.n_q);
    a.n_kv = static_cast<uint32_t>(p.n_kv);
    const AttnSplit sp = attn_split(p.n_seqs, p.n_heads, p.n_heads_kv, p.n_q, p.n_kv);
    a.groups = static_cast<uint32_t>(sp.groups);
    a.n_split = static_cast<uint32_t>(sp.n_split);
    a.split_len = static_cast<uint32_t>(sp.split_len);
    const int64_t blocks = p.n_seqs * p.n_heads_kv * sp.groups * int64_t(sp.n_split);
    const int64_t rows = p.n_seqs * p.n_q * p.n_heads;
    if (!grid_fits(blocks, kAttnThreads) || !grid_fits(rows, 64)) return hipErrorInvalidConfiguration;
    if constexpr (BF16)
        hipLaunchKernelGGL((attn_split_mma_kernel<D>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kAttnThreads), 0, stream, ATTN_ARGS(a));
    else
        hipLaunchKernelGGL((attn_split_kernel<D, false>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kAttnThreads), 0, stream, ATTN_ARGS(a));
    if (sp.n_split > 1) {
        hipLaunchKernelGGL((attn_combine_kernel<D, BF16>), dim3(static_cast<uint32_t>(rows)),
                           dim3(64), 0, stream, static_cast<const float *>(a.part), a.out, a.n_split);
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
