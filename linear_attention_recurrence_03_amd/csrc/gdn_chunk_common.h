// gdn_chunk_common.h -- device helpers shared by the chunked form's kernels
// (gdn_chunk.hip: the prep and the per-tile pass; gdn_chunk_head.hip: the whole-head
// pass; gdn_chunk_lag.hip: the two-chunk-lag pass).  Everything here has internal
// linkage: each translation unit gets its own copy.
//
// MFMA fragments.  An A operand (16 rows x 32 k) gives lane l row l%16 and eight
// k values; a B operand (32 k x 16 cols) gives lane l column l%16 and eight k
// values; the hardware pairs element j of lane group g = l/16 in A with the same
// element of B.  The accumulator gives lane l column l%16 and rows 4g..4g+3.
// Two stacked accumulator tiles therefore form a B operand directly if element
// j of group g stands for row 4g+j (j < 4) or 16+4g+j-4 (j >= 4) of the 32; every
// A operand here is loaded with that same k order, so no data moves between
// lanes when a product feeds the next one.
#pragma once

#include <atomic>

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

// ---- fragment blocks -------------------------------------------------------------
// A fragment block is the image of one 16-row x 32-k A operand, laid out so that
// each lane's fragment is one contiguous unit (its eight elements: 16 bytes for
// bf16, 32 for fp32) and a wave's read of the whole operand touches every LDS
// bank equally: the unit of row r for lane group g sits at position
// 4 r + (g ^ (r >> 2)).  Inside a unit the elements follow the fragment k order
// (4g+j for j < 4, 16+4g+j-4 for j >= 4), so the block multiplies B operands
// built from accumulator tiles.  The lower-triangular T and P are stored as the
// six blocks (row tile tt, k half h) with 32 h <= 16 tt + 15, in the order
// (0,0) (1,0) (2,0) (2,1) (3,0) (3,1); the other two are zero.
template <bool BF16>
constexpr int kFragBytes = BF16 ? 16 : 32;
template <bool BF16>
constexpr int kBlkBytes = 64 * kFragBytes<BF16>;

__device__ __forceinline__ int blk_unit(int r, int g) { return 4 * r + (g ^ (r >> 2)); }

template <bool BF16>
__device__ __forceinline__ Frag<BF16> frag_blk(const unsigned char *blk, int lane)
{
    return *reinterpret_cast<const Frag<BF16> *>(blk + kFragBytes<BF16> * blk_unit(lane & 15, lane >> 4));
}

// ---- workspace layout, per (seq, head, chunk) ----------------------------------
//   T     six fragment blocks (elements like q/k/v: fp32 or bf16)
//   P     six fragment blocks, holding P / sqrt(d)
//   gates [4][C] fp32: beta_r, e^{gam_r}, e^{gam_last - gam_r}, then e^{gam_last}
//                      repeated C times
// Rows past the end of a partial last chunk carry beta = e^gam = 0, so they add
// nothing to the state or to valid outputs.
template <bool BF16>
struct WsLayout {
    static constexpr int64_t kT = 0;
    static constexpr int64_t kP = 6 * kBlkBytes<BF16>;
    static constexpr int64_t kGates = 2 * kP;
    // gates: four rows of C floats (1 KiB); five with normalised q/k rows, which
    // then take a 2 KiB area
    static constexpr int64_t kBytes = kGates + 4 * C * 4;
    static constexpr int64_t kBytesNorm = kGates + 8 * C * 4;
    static constexpr int64_t stride(int l2norm_qk) { return l2norm_qk ? kBytesNorm : kBytes; }
};

// Workspace of the two-chunk-lag path (bf16 rows), per (seq, head, chunk):
//   T, P     six fragment blocks each, as above (P holds P / sqrt(d))
//   R1, R2   eight fragment blocks each (row tile tt, k half h) at 2 tt + h: the full
//            64 x 64 matrices R1 = -T diag(beta e^gam) K_n K_{n-1}^T and
//            R2 = -e^{c_{n-1}} T diag(beta e^gam) K_n K_{n-2}^T (zero when the
//            earlier chunk does not exist), bf16
//   gates    [8][C] fp32 rows: beta; e^gam; e^{gam_last - gam}; e^{gam_last}
//            repeated; e^gam for the output; rows 1 and 2 carry 1 / |k_r| and row 4
//            carries 1 / |q_r| when the op normalises q and k
struct WsLag {
    static constexpr int kBlk = kBlkBytes<true>;
    static constexpr int64_t kT = 0;
    static constexpr int64_t kP = 6 * kBlk;
    static constexpr int64_t kR1 = 12 * kBlk;
    static constexpr int64_t kR2 = 20 * kBlk;
    static constexpr int64_t kGates = 28 * kBlk;
    static constexpr int64_t kBytes = kGates + 8 * C * 4;
};

// A operand from rows of a padded row-major LDS matrix: lane (g, r) gets row
// row0 + r, k = k0 + 8g .. k0 + 8g + 7 (contiguous).
template <bool BF16>
__device__ __forceinline__ Frag<BF16> row_frag(const unsigned char *base, int stride, int row,
                                               int k0, int g)
{
    return *reinterpret_cast<const Frag<BF16> *>(base + row * stride + (k0 + 8 * g) * (BF16 ? 2 : 4));
}

constexpr int kPrepThreads = 256;

// LDS of the prep kernel (one workgroup per (seq, head, chunk)).  Region R holds
// the chunk's K rows (16-byte padded) while the products are formed; after that
// it is reused for T and A (as MFMA input type).  Q rows never pass through LDS:
// the two waves that form Q K^T load their row tiles straight into MFMA operand
// registers.
template <int D, bool BF16>
struct PrepSmem {
    using E = typename Elem<BF16>::T;
    static constexpr int ES = sizeof(E);
    static constexpr int RK = D * ES + 16;               // K, Q row stride (bytes)
    static constexpr int LDT = C + 16 / ES;              // T and A rows (elements)
    static constexpr int LDD = 16;                       // transposed diagonal blocks (floats)
    static constexpr int kMat = C * LDT * ES;            // one C x C matrix of E
    static constexpr int kK = 0;                         // during the products
    static constexpr int kT = 0, kAe = kMat;             // afterwards
    static constexpr int kR = (C * RK > 2 * kMat) ? C * RK : 2 * kMat;
    static constexpr int kD = kR;                        // 4 x [16][LDD] fp32
    static constexpr int kG = kD + 4 * 16 * LDD * 4;     // gates
    static constexpr int kN = kG + (4 * C + 4) * 4;      // 1/|k_r|, 1/|q_r| (normalised rows)
    static constexpr int kBytes = kN + 2 * C * 4;
    static constexpr int NBK = C * RK / 1024;            // DMA blocks of the K rows
    // Workgroups per CU that 160 KiB of LDS allows, at most five; the kernel's
    // register budget is set for that many (one wave per SIMD each).
    static constexpr int kPerCU = (160 * 1024 / kBytes < 5) ? 160 * 1024 / kBytes : 5;
    static_assert(C * RK % 1024 == 0 && kMat % 16 == 0 && kR % 16 == 0 && kPerCU >= 1, "layout");
};

// The output's factor 1/sqrt(d), applied where P is formed (and by the scan's
// output wave to e^gam), so that the output needs no scaling of its own.
template <int D>
constexpr float kOutScale = D == 32 ? 0.17677669529663687f : D == 64 ? 0.125f
                          : D == 96 ? 0.10206207261596575f : 0.08838834764831845f;

// Operand whose rows are columns c0 + (lane mod 16) of a row-major LDS matrix and
// whose k values are rows t0 + {4g..4g+3}, t0 + 16 + {4g..4g+3} (eight rows of
// one column).  bf16: two ds_read_b64_tr_b16; inside each group of 16 lanes
// this instruction hands lane i the (i mod 4)-th 16-bit value fetched by lane
// 4j + i/4 as its element j, so lane p fetches row t0 + 4g + p/4 (then 16 rows
// lower), columns c0 + 4 (p mod 4) .. +3.
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

// P = e^{gam_r - gam_s} (q_r . k_s) / sqrt(d) for s <= r (zero above the diagonal),
// for a pass that forms P itself from a chunk's K and Q rows in LDS (bf16, rows of
// `rk` bytes, k order 8g..8g+7 per lane group), written as the prep writes it: the
// ten lower 16 x 16 tiles, tile (tt, tc) as half tc % 2 of the fragment units of
// block (tt, tc / 2) of `pdst`.  The caller forms tiles first, first + step, ...;
// the products, scaling and rounding are the prep's, so P is identical bit for
// bit.  gam: the chunk's cumulative log gates.
template <int D>
__device__ __forceinline__ void form_p(const unsigned char *kb, const unsigned char *qb, int rk,
                                       const float *gam, unsigned char *pdst, int first, int step,
                                       int lane)
{
    const int gq = lane >> 4, cl = lane & 15;
    for (int i = first; i < 10; i += step) {
        const int tt = i < 1 ? 0 : i < 3 ? 1 : i < 6 ? 2 : 3;
        const int tc = i - tt * (tt + 1) / 2;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            acc = mma(row_frag<true>(kb, rk, 16 * tc + cl, 32 * ks, gq),
                      row_frag<true>(qb, rk, 16 * tt + cl, 32 * ks, gq), acc);
        const int row = 16 * tt + cl, col0 = 16 * tc + 4 * gq;
        const float g_row = gam[row];
        const float4 gc = *reinterpret_cast<const float4 *>(gam + col0);
        const float gcol[4] = {gc.x, gc.y, gc.z, gc.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float e = __expf(g_row - gcol[j]);
            acc[j] = (col0 + j <= row) ? kOutScale<D> * e * acc[j] : 0.f;
        }
        const int b = tt < 2 ? tt : 2 * tt - 2 + (tc >> 1);
        *reinterpret_cast<uint2 *>(pdst + b * kBlkBytes<true> + kFragBytes<true> * blk_unit(cl, gq) +
                                   8 * (tc & 1)) = make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
    }
}

// The halves of P's fragment units that form_p never writes (tiles (0, 1) and
// (2, 3), above the diagonal), set to zero.
__device__ __forceinline__ void zero_p_halves(unsigned char *pdst, int lane)
{
    const int u = kFragBytes<true> * blk_unit(lane & 15, lane >> 4) + 8;
    *reinterpret_cast<uint2 *>(pdst + u) = make_uint2(0u, 0u);
    *reinterpret_cast<uint2 *>(pdst + 3 * kBlkBytes<true> + u) = make_uint2(0u, 0u);
}

// A operand of K^T for state tile t in the permuted key order of the whole-head pass
// and the per-tile pass's U waves: row r is key 32 (t/2) + 8 (r/4) + 4 (t%2) + r%4,
// k is tokens t0 + 4g + j, t0 + 16 + 4g + j.  Two transposing reads: lane p of a group
// fetches row t0 + 4g + p/4 (then 16 rows lower) at keys kb + 8 (p mod 4) .. +3, and
// lane i receives the (i mod 4)-th value fetched by lane 4j + i/4.
__device__ __forceinline__ Frag<true> key_tr_frag(const unsigned char *base, int stride, int t0,
                                                   int t, int lane)
{
    const int g = lane >> 4, p = lane & 15;
    const int key = 32 * (t >> 1) + 4 * (t & 1) + 8 * (p & 3);
    const unsigned char *a1 = base + (t0 + 4 * g + (p >> 2)) * stride + 2 * key;
    typedef __attribute__((address_space(3))) short4_t lds_short4;
    const short4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(a1));
    const short4_t r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(a1 + 16 * stride));
    Frag<true> f;
    const uint2 u1 = __builtin_bit_cast(uint2, r1);
    const uint2 u2 = __builtin_bit_cast(uint2, r2);
    f.u = make_uint4(u1.x, u1.y, u2.x, u2.y);
    return f;
}

// Lower-triangular block matrix (six fragment blocks) times the 64-row B operand
// given as two k halves: rows tt of the product.
template <bool BF16>
__device__ __forceinline__ void tri_mul(const Frag<BF16> (&a)[6], const Frag<BF16> &b0,
                                        const Frag<BF16> &b1, floatx4 (&acc)[4])
{
    acc[0] = mma(a[0], b0, acc[0]);
    acc[1] = mma(a[1], b0, acc[1]);
    acc[2] = mma(a[3], b1, mma(a[2], b0, acc[2]));
    acc[3] = mma(a[5], b1, mma(a[4], b0, acc[3]));
}

// Raises the dynamic-LDS limit of `kern` to `bytes`, once per device (bit d of
// `done` records device d; concurrent first calls may both set it, harmlessly).
template <typename K>
hipError_t ensure_lds_limit(K kern, int bytes, std::atomic<uint64_t> &done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

// Phase timestamps of the trace build (-DGDN_PHASE_TRACE; off by default): the first
// kTraceGroups workgroups of a chunk-to-chunk pass record the shader clock at fixed
// points of their chunk steps (the per-tile pass in gdn_chunk.hip, the lag pass in
// gdn_chunk_lag.hip; linear_attention_recurrence_03_amd/phase_trace.py prints them).
constexpr int kTraceGroups = 8, kTracePhases = 1024;

}  // namespace
}  // namespace gdn
