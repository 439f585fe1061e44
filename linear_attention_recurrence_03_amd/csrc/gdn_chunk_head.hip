// gdn_chunk_head.hip -- the whole-head chunk-to-chunk pass of the chunked form
// (bf16 rows), for gfx950.  The chunk algebra and the prep kernel that writes T, P
// and the gate rows are in gdn_chunk.hip.
#include "gdn_chunk_common.h"

namespace gdn {
namespace {

// ---- the whole-head scan (bf16 rows) ------------------------------------------------
//
// One workgroup carries every value row of one (seq, head) through its chunks, so
// a chunk's shared operands (K, Q, T, P, gates) are brought into the compute unit
// once for all value rows instead of once per row block.  D / 16 waves (two per
// SIMD at D = 128) each own one value tile (16 rows) and do the whole chunk step
// for it with no hand-off between waves:
//   X = K M^T and (M Q^T) from the state's own accumulators, turned into bf16
//   operands in registers (the state's key order is permuted so that two stacked
//   accumulator tiles are a B operand with eight consecutive keys per lane);
//   E = beta V - beta e^gam X; Delta = T E; the output tile
//   O^T = e^gam (M Q^T) + Delta^T P^T stored from registers; and
//   M^T <- e^{gam_last} M^T + K^T diag(e^{gam_last - gam}) Delta (K^T from
//   transposing LDS reads that deliver the permuted key order).
// The chunk's data pass through two LDS slots: every wave copies a share of chunk
// n + 1 from global memory into registers during chunk n - 1 and writes it into
// the free slot at the end of chunk n, so one workgroup barrier per chunk suffices.
// A wave's registers then hold its own state rows, its operands and one staging
// share (171 at D = 128, two waves per SIMD); holding two value tiles per wave
// (four waves) halves the LDS operand reads but needs ~350 registers, and the
// copies between accumulation and vector registers that this forces made it slower
// (242 against 190 us per 4,096 x 32 call on MI355X).
//
// Row r of state tile t holds key 32 (t/2) + 8 (r/4) + 4 (t%2) + r%4.
template <int D>
struct HeadCfg {
    static constexpr int NVT = D / 16;                  // value tiles of a head
    static constexpr int NT = 1;                        // value tiles per wave
    static constexpr int NW = NVT / NT;                 // waves
    static constexpr int KT = D / 16, KS = D / 32;      // key tiles, 32-key steps
    static constexpr int RK = 2 * D + 32;               // K, Q, V row stride in LDS
    static_assert((RK / 16) % 4 == 2, "row stride");
    static constexpr int kK = 0, kQ = C * RK, kV = 2 * C * RK;
    static constexpr int kT = 3 * C * RK;               // T, P, gates as in the workspace
    static constexpr int kP = kT + 6 * kBlkBytes<true>;
    static constexpr int kG = kP + 6 * kBlkBytes<true>;
    static constexpr int kSlot = kG + 2048;
    static constexpr int kBytes = 2 * kSlot;
    static_assert(kBytes <= 160 * 1024, "LDS budget");
    // staging: per matrix (K, Q, V) PR = D/8 pieces of 16 bytes per row, spread over
    // the 64 NW lanes; then the workspace's T, P and gates (PIN: P in the workspace)
    // or its T and gates (P formed by the pass), in 16-byte pieces
    static constexpr int PR = D / 8;
    static constexpr int LANES = 64 * NW;
    static constexpr int RPS = LANES / PR;              // rows per staging round
    static constexpr int NR = C / RPS;                  // rounds per matrix
    static_assert(LANES % PR == 0 && C % RPS == 0, "staging rows");
    static constexpr int ws_pieces(bool pin)
    {
        return pin ? int(WsLayout<true>::kBytesNorm / 16) : (6 * kBlkBytes<true> + 2048) / 16;
    }
    static constexpr int nws(bool pin) { return (ws_pieces(pin) + LANES - 1) / LANES; }
    // byte offset of workspace piece i (the same offset in the LDS slot, from kT)
    static constexpr int ws_offset(bool pin, int i)
    {
        return (pin || 16 * i < 6 * kBlkBytes<true>) ? 16 * i : 16 * i + 6 * kBlkBytes<true>;
    }
    static constexpr int NSTAGE = 3 * NR + nws(true);
};

// One chunk's data in flight to LDS: each lane's 16-byte pieces (a native vector
// type, so that the array lives in registers).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <int D>
struct HeadStage {
    u32x4_t x[HeadCfg<D>::NSTAGE];
};

// Issues the loads of chunk m (nv valid rows) into st.
template <int D, bool PIN>
__device__ __forceinline__ void head_stage_load(HeadStage<D> &st, const unsigned char *k,
                                                const unsigned char *q, const unsigned char *v,
                                                const unsigned char *wsc, int64_t kq_bytes,
                                                int64_t hd_bytes, int m, int nv, int tid)
{
    using H = HeadCfg<D>;
    // wave-uniform chunk bases plus 32-bit lane offsets (64 token rows of all heads
    // span less than 4 GiB)
    const uint32_t row0 = tid / H::PR, col = (tid % H::PR) * 16;
    const uint32_t kqb = static_cast<uint32_t>(kq_bytes), hdb = static_cast<uint32_t>(hd_bytes);
    const unsigned char *kb = k + int64_t(m) * C * kq_bytes;
    const unsigned char *qb = q + int64_t(m) * C * kq_bytes;
    const unsigned char *vb = v + int64_t(m) * C * hd_bytes;
#pragma unroll
    for (int r = 0; r < H::NR; ++r) {
        const uint32_t row = min(row0 + r * H::RPS, uint32_t(nv - 1));
        st.x[r] = *reinterpret_cast<const u32x4_t *>(kb + (row * kqb + col));
        st.x[H::NR + r] = *reinterpret_cast<const u32x4_t *>(qb + (row * kqb + col));
        st.x[2 * H::NR + r] = *reinterpret_cast<const u32x4_t *>(vb + (row * hdb + col));
    }
#pragma unroll
    for (int r = 0; r < H::nws(PIN); ++r) {
        // pieces past the chunk's last re-read it and are not stored
        const int i = min(tid + r * H::LANES, H::ws_pieces(PIN) - 1);
        st.x[3 * H::NR + r] = *reinterpret_cast<const u32x4_t *>(wsc + H::ws_offset(PIN, i));
    }
}

// Writes the staged chunk into an LDS slot.
template <int D, bool PIN>
__device__ __forceinline__ void head_stage_store(const HeadStage<D> &st, unsigned char *slot,
                                                 int tid)
{
    using H = HeadCfg<D>;
    const int row0 = tid / H::PR, col = (tid % H::PR) * 16;
#pragma unroll
    for (int r = 0; r < H::NR; ++r) {
        const int off = (row0 + r * H::RPS) * H::RK + col;
        *reinterpret_cast<u32x4_t *>(slot + H::kK + off) = st.x[r];
        *reinterpret_cast<u32x4_t *>(slot + H::kQ + off) = st.x[H::NR + r];
        *reinterpret_cast<u32x4_t *>(slot + H::kV + off) = st.x[2 * H::NR + r];
    }
#pragma unroll
    for (int r = 0; r < H::nws(PIN); ++r) {
        const int i = tid + r * H::LANES;
        if (i < H::ws_pieces(PIN))
            *reinterpret_cast<u32x4_t *>(slot + H::kT + H::ws_offset(PIN, i)) = st.x[3 * H::NR + r];
    }
}

// The whole-head scan over chunks [c0, c1) of one (seq, head).  m_in: the state
// entering chunk c0 ([value][key] fp32, or null for zeros); m_out: where the state
// after chunk c1 - 1 goes.
template <int D, bool NORM>
__global__ __launch_bounds__(64 * HeadCfg<D>::NW) __attribute__((amdgpu_waves_per_eu(2)))
void chunk_head_kernel(const void *__restrict__ q, const void *__restrict__ k,
                       const void *__restrict__ v, const float *state_in, void *__restrict__ out,
                       float *state_out, const unsigned char *__restrict__ ws, int64_t n_tokens,
                       int64_t n_heads, int64_t n_k_heads, int n_chunks)
{
    using H = HeadCfg<D>;
    using W = WsLayout<true>;
    constexpr int NT = H::NT, KT = H::KT, KS = H::KS;
    // normalised rows keep P in the workspace (it needs the q row norms the prep
    // forms); plain rows have the pass form P from the K and Q rows it stages anyway
    constexpr bool PIN = NORM;
    constexpr int eg_row = NORM ? 4 : 1;
    extern __shared__ __align__(16) unsigned char smem[];

    const int64_t sh = blockIdx.x;
    const int64_t s = sh / n_heads, h = sh - s * n_heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gq = lane >> 4, cl = lane & 15;
    const int64_t kq_bytes = n_k_heads * D * 2, hd_bytes = n_heads * D * 2;
    const int64_t ktok0 = (s * n_tokens * n_k_heads + h % n_k_heads) * D;
    const int64_t tok0 = (s * n_tokens * n_heads + h) * D;
    const unsigned char *kp = static_cast<const unsigned char *>(k) + ktok0 * 2;
    const unsigned char *qp = static_cast<const unsigned char *>(q) + ktok0 * 2;
    const unsigned char *vp = static_cast<const unsigned char *>(v) + tok0 * 2;
    const int64_t ws_stride = W::kBytesNorm;   // the prep's stride for this pass
    const unsigned char *wsh = ws + sh * n_chunks * ws_stride;
    auto nv_of = [&](int m) { return static_cast<int>(min<int64_t>(C, n_tokens - int64_t(m) * C)); };
    const int nc = n_chunks;

    // state: Mt[i][t] = M[16 (wave NT + i) + cl][32 (t/2) + 8 gq + 4 (t%2) + j]
    floatx4 Mt[NT][KT];
    const int64_t st0 = sh * D * D;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int vrow = 16 * (wave * NT + i) + cl;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int key = 32 * (t >> 1) + 8 * gq + 4 * (t & 1);
            if (state_in) {
                const float4 m = *reinterpret_cast<const float4 *>(state_in + st0 + int64_t(vrow) * D + key);
                Mt[i][t] = floatx4{m.x, m.y, m.z, m.w};
            } else {
                Mt[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }

    if constexpr (!PIN) {
        // the zero halves of P, which no step writes
        if (wave == 0) {
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) zero_p_halves(smem + sl * H::kSlot + H::kP, lane);
        }
    }
    HeadStage<D> st;
    head_stage_load<D, PIN>(st, kp, qp, vp, wsh, kq_bytes, hd_bytes, 0, nv_of(0), tid);
    head_stage_store<D, PIN>(st, smem, tid);
    {
        const int m1 = min(1, nc - 1);
        head_stage_load<D, PIN>(st, kp, qp, vp, wsh + m1 * ws_stride, kq_bytes, hd_bytes, m1,
                                nv_of(m1), tid);
    }
    lds_barrier();

    uint16_t *obase = static_cast<uint16_t *>(out) + tok0;
    for (int n = 0; n < nc; ++n) {
        unsigned char *S = smem + (n & 1) * H::kSlot;
        const float *G = reinterpret_cast<const float *>(S + H::kG);
        if constexpr (!PIN) form_p<D>(S + H::kK, S + H::kQ, H::RK, G + 5 * C, S + H::kP, wave, H::NW, lane);
        // the state entering chunk n as bf16 operands (B of M^T, A of M)
        Frag<true> mb[NT][KS];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mb[i][ks] = acc_frag<true>(Mt[i][2 * ks], Mt[i][2 * ks + 1]);
        // X = K M^T
        floatx4 X[NT][4];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) X[i][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            Frag<true> kf[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) kf[tt] = row_frag<true>(S + H::kK, H::RK, 16 * tt + cl, 32 * ks, gq);
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) X[i][tt] = mma(kf[tt], mb[i][ks], X[i][tt]);
        }
        // E = beta V - beta e^gam X; Delta = T E
        Frag<true> tf[6];
#pragma unroll
        for (int b = 0; b < 6; ++b) tf[b] = frag_blk<true>(S + H::kT + b * kBlkBytes<true>, lane);
        floatx4 dl[NT][4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int r = 16 * tt + 4 * gq;
            const float4 b4 = *reinterpret_cast<const float4 *>(G + r);
            const float4 e4 = *reinterpret_cast<const float4 *>(G + C + r);
            const floatx4 bb = floatx4{b4.x, b4.y, b4.z, b4.w};
            const floatx4 be = bb * floatx4{e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const floatx4 vv = col4<true>(S + H::kV, H::RK, 16 * tt, 16 * (wave * NT + i), lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) X[i][tt][j] = fmaf(-be[j], X[i][tt][j], bb[j] * vv[j]);
            }
        }
#pragma unroll
        for (int i = 0; i < NT; ++i) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) dl[i][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
            tri_mul<true>(tf, acc_frag<true>(X[i][0], X[i][1]), acc_frag<true>(X[i][2], X[i][3]), dl[i]);
        }
        // output: O^T = e^gam (M Q^T) + Delta^T P^T (1/sqrt(d) in e^gam and P)
        floatx4 O[NT][4];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) O[i][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            Frag<true> qf[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) qf[tt] = row_frag<true>(S + H::kQ, H::RK, 16 * tt + cl, 32 * ks, gq);
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) O[i][tt] = mma(mb[i][ks], qf[tt], O[i][tt]);
        }
        if constexpr (!PIN) lds_barrier();   // P formed by every wave
        Frag<true> pf[6];
#pragma unroll
        for (int b = 0; b < 6; ++b) pf[b] = frag_blk<true>(S + H::kP + b * kBlkBytes<true>, lane);
        float eg[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) eg[tt] = kOutScale<D> * G[eg_row * C + 16 * tt + cl];
        const int nv = nv_of(n);
        uint16_t *ob = obase + int64_t(n) * C * (hd_bytes / 2);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const Frag<true> d0 = acc_frag<true>(dl[i][0], dl[i][1]);
            const Frag<true> d1 = acc_frag<true>(dl[i][2], dl[i][3]);
            floatx4 a[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) a[tt] = O[i][tt] * eg[tt];
            a[0] = mma(d0, pf[0], a[0]);
            a[1] = mma(d0, pf[1], a[1]);
            a[2] = mma(d1, pf[3], mma(d0, pf[2], a[2]));
            a[3] = mma(d1, pf[5], mma(d0, pf[4], a[3]));
            const int c0 = 16 * (wave * NT + i) + 4 * gq;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                if (nv == C || 16 * tt + cl < nv)
                    *reinterpret_cast<uint2 *>(ob + (16 * tt + cl) * (hd_bytes / 2) + c0) =
                        make_uint2(pack2(a[tt][0], a[tt][1]), pack2(a[tt][2], a[tt][3]));
            }
        }
        floatx4 ed[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const float4 d4 = *reinterpret_cast<const float4 *>(G + 2 * C + 16 * tt + 4 * gq);
            ed[tt] = floatx4{d4.x, d4.y, d4.z, d4.w};
        }
        const float ec = G[3 * C];
        // M^T <- e^{gam_last} M^T + K^T diag(e^{gam_last - gam}) Delta
        Frag<true> dt[NT][2];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            dt[i][0] = acc_frag<true>(ed[0] * dl[i][0], ed[1] * dl[i][1]);
            dt[i][1] = acc_frag<true>(ed[2] * dl[i][2], ed[3] * dl[i][3]);
        }
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const Frag<true> k0 = key_tr_frag(S + H::kK, H::RK, 0, t, lane);
            const Frag<true> k1 = key_tr_frag(S + H::kK, H::RK, 32, t, lane);
#pragma unroll
            for (int i = 0; i < NT; ++i) Mt[i][t] = mma(k1, dt[i][1], mma(k0, dt[i][0], Mt[i][t] * ec));
        }
        // chunk n + 1 into the other slot, then the loads of chunk n + 2 (the last
        // chunk again near the end: loaded, never stored)
        if (n + 1 < nc) head_stage_store<D, PIN>(st, smem + ((n + 1) & 1) * H::kSlot, tid);
        const int m2 = min(n + 2, nc - 1);
        head_stage_load<D, PIN>(st, kp, qp, vp, wsh + m2 * ws_stride, kq_bytes, hd_bytes, m2,
                                nv_of(m2), tid);
        lds_barrier();
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int vrow = 16 * (wave * NT + i) + cl;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int key = 32 * (t >> 1) + 8 * gq + 4 * (t & 1);
            *reinterpret_cast<float4 *>(state_out + st0 + int64_t(vrow) * D + key) =
                make_float4(Mt[i][t][0], Mt[i][t][1], Mt[i][t][2], Mt[i][t][3]);
        }
    }
}

// The whole-head pass: one workgroup per (seq, head), D / 16 waves.
template <int D, bool NORM>
hipError_t launch_head(const Problem &p, const unsigned char *ws, int n_chunks, hipStream_t stream)
{
    using H = HeadCfg<D>;
    auto kern = chunk_head_kernel<D, NORM>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = ensure_lds_limit(kern, H::kBytes, lds_set);
    if (e != hipSuccess) return e;
    const int64_t blocks = p.n_seqs * p.n_heads;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(64 * H::NW), H::kBytes,
                       stream, p.q, p.k, p.v, p.state_in, p.out, p.state_out, ws, p.n_tokens,
                       p.n_heads, p.n_k_heads, n_chunks);
    return hipGetLastError();
}

template <int D>
hipError_t launch_head_d(const Problem &p, const unsigned char *ws, int n_chunks, hipStream_t stream)
{
    return p.l2norm_qk ? launch_head<D, true>(p, ws, n_chunks, stream)
                       : launch_head<D, false>(p, ws, n_chunks, stream);
}

}  // namespace

bool head_pass_fits(int64_t n_sh, int head_dim) { return grid_fits(n_sh, 4 * int64_t(head_dim)); }

hipError_t launch_head_pass(const Problem &p, const unsigned char *ws, int n_chunks,
                            hipStream_t stream)
{
    switch (p.head_dim) {
    case 32: return launch_head_d<32>(p, ws, n_chunks, stream);
    case 64: return launch_head_d<64>(p, ws, n_chunks, stream);
    case 96: return launch_head_d<96>(p, ws, n_chunks, stream);
    case 128: return launch_head_d<128>(p, ws, n_chunks, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
