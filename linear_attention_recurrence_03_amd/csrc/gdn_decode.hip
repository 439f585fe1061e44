// gdn_decode.hip -- token recurrence of the gated delta rule for gfx950.
//
// The step (per sequence, head and token; state M stored [value][key]):
//     M <- exp(g) M;  delta = beta (v - M k);  M <- M + delta k^T;
//     out = M q / sqrt(d)
// ("Gated Delta Net on AMD", velstech.net, section "What Gated Delta Net is,
// in plain language": a gate on the state and a delta-rule overwrite; state
// layout, log-domain g and the 1/sqrt(head_dim) scaling from the "ggml
// attention kernels" model card, contract notes under "Shapes, in torch
// order").
//
// Value rows of M are independent given (k, q, g, beta) of the token, so each
// state row is one unit of work.  A row of d fp32 values is held by LPR = 32 or
// 16 lanes with d/LPR consecutive values each (the width rule of the model
// card's supports predicate: d a multiple of 32), so one wave64 load instruction
// covers 64/LPR adjacent rows -- contiguous bytes, fully coalesced.  A wave keeps
// (64/LPR)*NP rows in registers for the whole call: the state is read once and
// written once, which is all of the HBM traffic that matters (the model card
// notes that a 2 MB state copy per layer per token is most of the cost).  Per
// token each row needs two dot products over its keys (M_i.k and M_i.q), done as
// lane partials plus a DPP reduction over the row's lanes (and a swizzle across
// the two 16-lane rows of a half-wave at LPR = 32); k.q is reduced alongside.
// Since M_new q = exp(g) M q + delta (k.q), the readout needs no second pass
// over the row.
#include <type_traits>

#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kWaves = 4;   // waves per workgroup

// One state row of zeros (the widest head): a call without an initial state reads
// its rows from here, so that the state loads are unconditional and no branch
// joins them (a join makes the compiler wait for them before anything else issues).
__device__ float kZeroRow[128] = {};

template <int NV>
struct Vec {
    float x[NV];
};

template <int NV>
__device__ __forceinline__ Vec<NV> load_f32(const float *p)
{
    // a lane's NV floats start at a multiple of NV floats: 16-byte pieces when NV is
    // a multiple of four, 8-byte ones when it is even
    Vec<NV> r;
    if constexpr (NV % 4 == 0) {
#pragma unroll
        for (int j = 0; j < NV / 4; ++j) {
            const float4 t = reinterpret_cast<const float4 *>(p)[j];
            r.x[4 * j] = t.x; r.x[4 * j + 1] = t.y; r.x[4 * j + 2] = t.z; r.x[4 * j + 3] = t.w;
        }
    } else if constexpr (NV % 2 == 0) {
#pragma unroll
        for (int j = 0; j < NV / 2; ++j) {
            const float2 t = reinterpret_cast<const float2 *>(p)[j];
            r.x[2 * j] = t.x; r.x[2 * j + 1] = t.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) r.x[i] = p[i];
    }
    return r;
}

template <int NV>
__device__ __forceinline__ void store_f32(float *p, const Vec<NV> &r)
{
    if constexpr (NV % 4 == 0) {
#pragma unroll
        for (int j = 0; j < NV / 4; ++j)
            reinterpret_cast<float4 *>(p)[j] =
                make_float4(r.x[4 * j], r.x[4 * j + 1], r.x[4 * j + 2], r.x[4 * j + 3]);
    } else if constexpr (NV % 2 == 0) {
#pragma unroll
        for (int j = 0; j < NV / 2; ++j)
            reinterpret_cast<float2 *>(p)[j] = make_float2(r.x[2 * j], r.x[2 * j + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) p[i] = r.x[i];
    }
}

// NW 32-bit words from p, which is aligned to 16 bytes when NW is a multiple of four
// and to 8 when NW is even (a lane's slice of NV = 2 NW bf16 values)
template <int NW>
__device__ __forceinline__ void load_words(const char *p, uint32_t (&w)[NW])
{
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int j = 0; j < NW / 4; ++j) {
            const uint4 t = reinterpret_cast<const uint4 *>(p)[j];
            w[4 * j] = t.x; w[4 * j + 1] = t.y; w[4 * j + 2] = t.z; w[4 * j + 3] = t.w;
        }
    } else if constexpr (NW % 2 == 0) {
#pragma unroll
        for (int j = 0; j < NW / 2; ++j) {
            const uint2 t = reinterpret_cast<const uint2 *>(p)[j];
            w[2 * j] = t.x; w[2 * j + 1] = t.y;
        }
    } else {
#pragma unroll
        for (int j = 0; j < NW; ++j) w[j] = reinterpret_cast<const uint32_t *>(p)[j];
    }
}

template <int NV, bool BF16>
__device__ __forceinline__ Vec<NV> load_in(const void *base, int64_t off)
{
    if constexpr (!BF16) {
        return load_f32<NV>(static_cast<const float *>(base) + off);
    } else {
        const uint16_t *p = static_cast<const uint16_t *>(base) + off;
        Vec<NV> r;
        if constexpr (NV % 2 == 0) {
            uint32_t w[NV / 2];
            load_words<NV / 2>(reinterpret_cast<const char *>(p), w);
#pragma unroll
            for (int j = 0; j < NV / 2; ++j) {
                r.x[2 * j] = __uint_as_float(w[j] << 16);
                r.x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) r.x[i] = bf16_to_f32(p[i]);
        }
        return r;
    }
}

// A copy of x in a register other than x's own (early-clobber output), made at this
// point of the program: once a loaded value has been copied, the next load can
// land in its register while the copy is in use, and no copy of a load still in
// flight is ever needed.
__device__ __forceinline__ float fresh(float x)
{
    float y;
    asm volatile("v_mov_b32 %0, %1" : "=&v"(y) : "v"(x) : "memory");
    return y;
}

// x, computed from loaded bits, fixed at this point of the program: its inputs are
// dead from here on, and no later load is moved above it.
__device__ __forceinline__ float pin(float x)
{
    asm volatile("" : "+v"(x) : : "memory");
    return x;
}

// A token's q or k slice as loaded (bf16: the raw bits), converted when used, so
// that the next token's loads can be in flight across the current token's work.
template <int NV, bool BF16>
struct RawIn;
template <int NV>
struct RawIn<NV, false> {
    Vec<NV> x;
};
template <int NV>
struct RawIn<NV, true> {
    // The aligned 32-bit words that hold the slice (two values each). An odd width
    // starts at the high half of its first word on odd lanes (odd = 1), and reads one
    // value past its end on even lanes: in bounds, as 32 lanes cover the whole row.
    uint32_t w[(NV + 1) / 2];
    uint32_t odd;
};

// The raw loads take a token's row start (the same in every lane) and a lane's
// 32-bit offset in elements.
template <int NV, bool BF16>
__device__ __forceinline__ RawIn<NV, BF16> load_raw(const void *base, uint32_t off)
{
    // byte offsets formed in 32 bits, so that the address is base + zero-extended offset
    const char *b = static_cast<const char *>(base);
    RawIn<NV, BF16> r;
    if constexpr (!BF16) {
        r.x = load_f32<NV>(reinterpret_cast<const float *>(b + off * 4u));
    } else {
        if constexpr (NV % 2 == 0) {
            load_words<NV / 2>(b + off * 2u, r.w);
        } else {
            const uint32_t *pw = reinterpret_cast<const uint32_t *>(b + (off >> 1) * 4u);
#pragma unroll
            for (int j = 0; j < (NV + 1) / 2; ++j) r.w[j] = pw[j];
            r.odd = off & 1u;
        }
    }
    return r;
}

template <int NV, bool BF16>
__device__ __forceinline__ Vec<NV> cvt_in(const RawIn<NV, BF16> &r)
{
    if constexpr (!BF16) {
        Vec<NV> v;
#pragma unroll
        for (int i = 0; i < NV; ++i) v.x[i] = fresh(r.x.x[i]);
        return v;
    } else {
        // half j of the words as a float
        auto half = [&](int j) {
            return __uint_as_float((j & 1) ? (r.w[j >> 1] & 0xffff0000u) : (r.w[j >> 1] << 16));
        };
        Vec<NV> v;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if constexpr (NV % 2 == 0)
                v.x[i] = pin(half(i));
            else
                v.x[i] = pin(r.odd ? half(i + 1) : half(i));
        }
        return v;
    }
}

// One v element as loaded: bf16 loads the aligned 32-bit pair that holds it (in
// bounds: rows have an even width), so no narrow load needs widening later.
template <bool BF16>
using RawScalar = typename std::conditional<BF16, uint32_t, float>::type;

template <bool BF16>
__device__ __forceinline__ RawScalar<BF16> load_scalar_raw(const void *base, uint32_t off)
{
    const char *b = static_cast<const char *>(base);
    if constexpr (BF16)
        return *reinterpret_cast<const uint32_t *>(b + (off >> 1) * 4u);
    else
        return *reinterpret_cast<const float *>(b + off * 4u);
}

// sh: 16 when the element is the pair's low half (an even offset), else 0
template <bool BF16>
__device__ __forceinline__ float cvt_scalar(RawScalar<BF16> x, uint32_t sh)
{
    if constexpr (BF16)
        return pin(__uint_as_float((x << sh) & 0xffff0000u));
    else
        return fresh(x);
}

template <bool BF16>
__device__ __forceinline__ float load_scalar_in(const void *base, int64_t off)
{
    if constexpr (BF16)
        return bf16_to_f32(static_cast<const uint16_t *>(base)[off]);
    else
        return static_cast<const float *>(base)[off];
}

template <bool BF16>
__device__ __forceinline__ void store_scalar_out(void *base, int64_t off, float x)
{
    if constexpr (BF16)
        static_cast<uint16_t *>(base)[off] = f32_to_bf16(x);
    else
        static_cast<float *>(base)[off] = x;
}

// element e of a bf16 (BF16) or fp32 array, as a byte pointer
template <bool BF16>
__device__ __forceinline__ const char *elem(const void *base, int64_t e)
{
    return static_cast<const char *>(base) + e * (BF16 ? 2 : 4);
}

// Sum over the L lanes of a row: 16 lanes (one DPP row) in four DPP steps, 32 with
// a swizzle across the two rows of a half-wave besides.
template <int L>
__device__ __forceinline__ float sum_lanes(float x)
{
    if constexpr (L == 32) {
        return sum32(x);
    } else {
        x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
        x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
        x += dpp_mov<0x141>(x);  // row_half_mirror
        x += dpp_mov<0x140>(x);  // row_mirror
        return x;
    }
}

// One workgroup = kWaves waves = kWaves*(64/LPR)*NP consecutive value rows of one
// (seq, head).  Grid: n_seqs * n_heads * (D / rows_per_block) workgroups.
// Everything the first loads need comes first, in 14 dwords: this file is built to
// have the hardware preload them into scalar registers at wave launch, so the
// state and token loads go out without waiting on argument loads (the kernel's
// life at one token per call is a few such round trips).  With PK the token
// count (< 2^31) and both head counts (< 2^16) are packed into two of them
// (tok32, heads16); otherwise the full-width counts further on are used and read
// like any argument.  Head counts fit in 32 bits: the grid, one workgroup per
// group of rows of each (seq, head), does.  ONE: the call has a single token
// (straight-line code); otherwise a software pipeline keeps two tokens' inputs in
// flight.
template <int D, int LPR, int NP, bool BF16, bool PK, bool ONE>
__global__ __launch_bounds__(kWaves * 64) void recurrent_kernel(
    const void *__restrict__ k, const void *__restrict__ q, const float *state_in,
    const void *__restrict__ v, const float *__restrict__ g, const float *__restrict__ beta,
    uint32_t tok32, uint32_t heads16, int64_t n_tokens_full, int n_heads_full,
    int n_k_heads_full, void *__restrict__ out, float *state_out, float scale, int l2norm_qk,
    int raw_gates)
{
    const int64_t n_tokens = PK ? int64_t(tok32) : n_tokens_full;
    const int n_heads32 = PK ? int(heads16 & 0xffffu) : n_heads_full;
    const int n_k_heads32 = PK ? int(heads16 >> 16) : n_k_heads_full;
    const int64_t n_heads = n_heads32, n_k_heads = n_k_heads32;
    static_assert(LPR == 16 || LPR == 32, "a row spans 16 or 32 lanes");
    constexpr int NV = D / LPR;          // keys per lane
    constexpr int G = 64 / LPR;          // rows side by side in a wave
    constexpr int kRowsPerWave = G * NP;
    constexpr int kRowsPerBlock = kWaves * kRowsPerWave;
    constexpr int kBlocksPerHead = D / kRowsPerBlock;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = (lane & (LPR - 1)) * NV;
    const uint32_t shu = blockIdx.x / kBlocksPerHead;   // s * n_heads + h
    const int rb = blockIdx.x % kBlocksPerHead;
    const uint32_t su = shu / static_cast<uint32_t>(n_heads32);
    const uint32_t hu = shu - su * static_cast<uint32_t>(n_heads32);
    const int64_t sh = shu, s = su, h = hu;
    // rows of this lane: row0 + G p, p < NP (the wave's G groups of LPR lanes interleave)
    const int row0 = rb * kRowsPerBlock + wave * kRowsPerWave + (lane >> (LPR == 16 ? 4 : 5));
    const int64_t st_base = sh * D * D;

    static_assert(D <= 128, "the zero row covers head_dim <= 128");
    Vec<NV> M[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const float *row = state_in ? state_in + st_base + (int64_t)(row0 + G * p) * D : kZeroRow;
        M[p] = load_f32<NV>(row + col);
    }

    // token t of (s, h): v and out at ((s*T + t)*H + h)*D, gates at (s*T + t)*H + h,
    // q and k at ((s*T + t)*Hk + h % Hk)*D
    int64_t gi = s * n_tokens * n_heads + h;
    int64_t ki = s * n_tokens * n_k_heads + hu % static_cast<uint32_t>(n_k_heads32);
    // One token of (s, h): decay, delta update and read-out of the rows held here,
    // with out at token offset go.
    auto token = [&](Vec<NV> kv, Vec<NV> qv, const float *vr, float gt, float bt, int64_t go) {
        if (l2norm_qk) {
            // every row's lanes hold the whole k and q rows: one reduction each
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                sk = fmaf(kv.x[i], kv.x[i], sk);
                sq = fmaf(qv.x[i], qv.x[i], sq);
            }
            const float rk = 1.f / sqrtf(sum_lanes<LPR>(sk) + kL2Eps);
            const float rq = 1.f / sqrtf(sum_lanes<LPR>(sq) + kL2Eps);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                kv.x[i] *= rk;
                qv.x[i] *= rq;
            }
        }
        if (raw_gates) {
            gt = neg_softplus(gt);
            bt = sigmoid(bt);
        }
        const float alpha = __expf(gt);
        char *const orow = static_cast<char *>(out) + go * D * (BF16 ? 2 : 4);   // token's out row
        float a[NP], b[NP], kq = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) kq = fmaf(kv.x[i], qv.x[i], kq);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            a[p] = 0.f;
            b[p] = 0.f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                a[p] = fmaf(M[p].x[i], kv.x[i], a[p]);
                b[p] = fmaf(M[p].x[i], qv.x[i], b[p]);
            }
        }
        kq = sum_lanes<LPR>(kq);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            a[p] = sum_lanes<LPR>(a[p]);
            b[p] = sum_lanes<LPR>(b[p]);
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            // retrieval from the gated state: (alpha M) k = alpha (M k)
            const float delta = bt * (vr[p] - alpha * a[p]);
#pragma unroll
            for (int i = 0; i < NV; ++i) M[p].x[i] = fmaf(alpha, M[p].x[i], delta * kv.x[i]);
            const float o = scale * fmaf(alpha, b[p], delta * kq);
            if ((lane & (LPR - 1)) == 0) {
                char *dst = orow + static_cast<uint32_t>(row0 + G * p) * (BF16 ? 2u : 4u);
                if constexpr (BF16)
                    *reinterpret_cast<uint16_t *>(dst) = f32_to_bf16(o);
                else
                    *reinterpret_cast<float *>(dst) = o;
            }
        }
    };

    if constexpr (ONE) {
        // a single token: straight-line loads, the gates through the scalar path
        float vr[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) vr[p] = load_scalar_in<BF16>(v, gi * D + row0 + G * p);
        token(load_in<NV, BF16>(k, ki * D + col), load_in<NV, BF16>(q, ki * D + col), vr, g[gi],
              beta[gi], gi);
    } else {
        // Two tokens in flight: stages A and B hold the raw bits of the next two
        // tokens' inputs. Each stage is converted, then at once reloaded with the
        // token two places on, and only then is its token worked on, so a load has
        // two tokens' arithmetic to land. The loop handles two tokens per pass, so
        // that no register of an in-flight load is ever copied (a copy would wait
        // for it). The gates go through the vector path (a lane-varying zero
        // offset) so that the waits on the cross-lane sums never also wait on them.
        int zoff;
        asm volatile("v_mov_b32 %0, 0" : "=v"(zoff));
        struct Raw {
            RawIn<NV, BF16> k, q;
            RawScalar<BF16> v[NP];
            float g, b;
        };
        const int64_t gi0 = gi, ki0 = ki;
        const uint32_t vsh = (row0 & 1) ? 0u : 16u;   // rows row0 + G p share row0's parity
        const uint32_t colu = static_cast<uint32_t>(col), zoff4 = static_cast<uint32_t>(zoff) * 4u;
        auto fetch = [&](int64_t t) {
            const int64_t gx = gi0 + t * n_heads, kx = ki0 + t * n_k_heads;
            Raw r;
            r.k = load_raw<NV, BF16>(elem<BF16>(k, kx * D), colu);
            r.q = load_raw<NV, BF16>(elem<BF16>(q, kx * D), colu);
            const char *vrow = elem<BF16>(v, gx * D);
#pragma unroll
            for (int p = 0; p < NP; ++p)
                r.v[p] = load_scalar_raw<BF16>(vrow, static_cast<uint32_t>(row0 + G * p));
            r.g = *reinterpret_cast<const float *>(elem<false>(g, gx) + zoff4);
            r.b = *reinterpret_cast<const float *>(elem<false>(beta, gx) + zoff4);
            return r;
        };
        struct Tok {
            Vec<NV> k, q;
            float v[NP];
            float g, b;
        };
        auto convert = [&](const Raw &r) {
            Tok c;
            c.k = cvt_in<NV, BF16>(r.k);
            c.q = cvt_in<NV, BF16>(r.q);
#pragma unroll
            for (int p = 0; p < NP; ++p) c.v[p] = cvt_scalar<BF16>(r.v[p], vsh);
            c.g = fresh(r.g);
            c.b = fresh(r.b);
            return c;
        };
        const int64_t last = n_tokens - 1;
        Raw A = fetch(0);
        Raw B = fetch(last < 1 ? last : 1);
        int64_t t = 0;
        for (; t + 2 < n_tokens; t += 2) {
            const Tok ca = convert(A);
            A = fetch(t + 2);
            token(ca.k, ca.q, ca.v, ca.g, ca.b, gi0 + t * n_heads);
            const Tok cb = convert(B);
            B = fetch(t + 3 < last ? t + 3 : last);   // past the end: the last token again
            token(cb.k, cb.q, cb.v, cb.g, cb.b, gi0 + (t + 1) * n_heads);
        }
        // one or two tokens left, in A and B
        const Tok ca = convert(A);
        token(ca.k, ca.q, ca.v, ca.g, ca.b, gi0 + t * n_heads);
        if (t + 1 < n_tokens) {
            const Tok cb = convert(B);
            token(cb.k, cb.q, cb.v, cb.g, cb.b, gi0 + (t + 1) * n_heads);
        }
    }

#pragma unroll
    for (int p = 0; p < NP; ++p)
        store_f32<NV>(state_out + st_base + (int64_t)(row0 + G * p) * D + col, M[p]);
}

template <int D, int LPR, int NP, bool BF16, bool ONE>
hipError_t launch_rec(const Problem &p, hipStream_t stream)
{
    const bool pk = p.n_tokens < (int64_t(1) << 31) && p.n_heads < (1 << 16) &&
                    p.n_k_heads < (1 << 16);
    constexpr int kRowsPerBlock = kWaves * (64 / LPR) * NP;
    static_assert(D % kRowsPerBlock == 0, "rows per block must divide head_dim");
    const int64_t blocks = p.n_seqs * p.n_heads * (D / kRowsPerBlock);
    if (!grid_fits(blocks, kWaves * 64)) return hipErrorInvalidConfiguration;
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    const uint32_t tok32 = pk ? static_cast<uint32_t>(p.n_tokens) : 0u;
    const uint32_t heads16 = pk ? static_cast<uint32_t>(p.n_heads | (p.n_k_heads << 16)) : 0u;
    auto kern = pk ? recurrent_kernel<D, LPR, NP, BF16, true, ONE>
                   : recurrent_kernel<D, LPR, NP, BF16, false, ONE>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(kWaves * 64), 0, stream,
                       p.k, p.q, p.state_in, p.v, p.g, p.beta, tok32, heads16, p.n_tokens,
                       static_cast<int>(p.n_heads), static_cast<int>(p.n_k_heads), p.out,
                       p.state_out, scale, p.l2norm_qk, p.raw_gates);
    return hipGetLastError();
}

// Lanes per row and rows per wave. A single token: 32 lanes per row, 8 rows per
// wave (NP = 4) once there are enough rows to fill the chip with workgroups, else 4
// (NP = 2: half as many waves, each issuing two state loads; 3.71 against 3.94 us
// per layer for 1 x 32 heads, d = 128); 16 lanes per row measured slower there
// (3.62 against 3.56 us, batched 50.1 against 48.2). Several tokens are bound by
// each wave's instructions per token: from 8192 rows, 16 lanes per row (no swizzle
// in the reductions, half the per-row share of converting and reducing k and q)
// with 4 rows per wave, and 8 from 16384 (32 tokens, d = 128, bf16: 16.4 against
// 20.1 us at 8192 rows, 23.9 against 30.8 at 16384, 40.7 against 50.6 at 32768);
// below 8192 rows, 32 lanes and 2 rows per wave keep twice the waves in flight
// (14.5 against 14.8 us at 4096 rows).
template <int D, bool BF16>
hipError_t launch_rec_d(const Problem &p, hipStream_t stream)
{
    const int64_t rows = p.n_seqs * p.n_heads * D;
    if (p.n_tokens == 1)
        return rows >= 256 * 32 * 4 ? launch_rec<D, 32, 4, BF16, true>(p, stream)
                                    : launch_rec<D, 32, 2, BF16, true>(p, stream);
    if (rows >= 16384) return launch_rec<D, 16, 2, BF16, false>(p, stream);
    if (rows >= 8192) return launch_rec<D, 16, 1, BF16, false>(p, stream);
    return launch_rec<D, 32, 1, BF16, false>(p, stream);
}

template <bool BF16>
hipError_t launch_rec_t(const Problem &p, hipStream_t stream)
{
    switch (p.head_dim) {
    case 32: return launch_rec_d<32, BF16>(p, stream);
    case 64: return launch_rec_d<64, BF16>(p, stream);
    case 96: return launch_rec_d<96, BF16>(p, stream);
    case 128: return launch_rec_d<128, BF16>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

// Copies (or zeroes) count4 float4s: the state is a whole number of 16-byte
// groups (head_dim^2 floats per head) at 16-byte aligned addresses.
__global__ __launch_bounds__(256) void state_copy_kernel(const float4 *__restrict__ src,
                                                         float4 *__restrict__ dst,
                                                         int64_t count4)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count4;
         i += stride)
        dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_recurrent(const Problem &p, hipStream_t stream)
{
    return p.bf16 ? launch_rec_t<true>(p, stream) : launch_rec_t<false>(p, stream);
}

hipError_t launch_state_copy(const float *state_in, float *state_out, int64_t count,
                             hipStream_t stream)
{
    if (count <= 0) return hipSuccess;
    const int64_t count4 = count / 4;   // count = n_seqs * n_heads * head_dim^2, head_dim % 32 == 0
    int64_t blocks = (count4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(state_copy_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       stream, reinterpret_cast<const float4 *>(state_in),
                       reinterpret_cast<float4 *>(state_out), count4);
    return hipGetLastError();
}

}  // namespace gdn
