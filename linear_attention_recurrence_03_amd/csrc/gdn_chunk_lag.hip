// gdn_chunk_lag.hip -- the two-chunk-lag chunk-to-chunk pass of the chunked form
// (bf16 rows, GDN_ALGO_CHUNKED_LAG), for gfx950.  Its prep variant (the cross-chunk
// matrices R1, R2) is the LAG instance of the prep kernel in gdn_chunk.hip.
#include "gdn_chunk_common.h"

namespace gdn {
namespace {

// Lag pass timestamps (trace builds only): for waves C, G, U, O and each phase,
// after the barrier that opens it (slot 0), once the wave's operands have landed
// (slot 1; the wave then waits for them explicitly) and before the barrier that
// closes it (slot 2); gdn_phase_trace_read copies them out.
#ifdef GDN_PHASE_TRACE
__device__ uint64_t g_phase_trace[kTraceGroups][4][kTracePhases][3];
#endif

struct LagTrace {
    int wg, wave;
    __device__ __forceinline__ void mark(int t, int slot, int lane) const
    {
#ifdef GDN_PHASE_TRACE
        const int p = t + 1;   // phases -1 .. n_chunks at 0 ..
        if (wg < kTraceGroups && lane == 0 && p < kTracePhases)
            g_phase_trace[wg][wave][p][slot] = __builtin_amdgcn_s_memtime();
#else
        (void)t;
        (void)slot;
        (void)lane;
#endif
    }
    // operands landed: an explicit wait only when tracing (the compiler places its
    // own waits otherwise).  The opening stamp's store, issued last, may stay in
    // flight: its acknowledgement is not what is measured.
    __device__ __forceinline__ void landed(int t, int lane) const
    {
#ifdef GDN_PHASE_TRACE
        wait_vmem_le<1>();
        mark(t, 1, lane);
#else
        (void)t;
        (void)lane;
#endif
    }
};

// ---- the two-chunk-lag scan (bf16 rows) --------------------------------------------
//
// With S_n the state entering chunk n (value rows x key columns), c_n the gate sum
// of chunk n and Dt_n = diag(e^{c_n - gam}) Delta_n the scaled deltas the state
// update uses, writing S_n = e^{c_{n-1}} S_{n-1} + Dt_{n-1}^T K_{n-1} twice gives
//
//   Delta_n = T_n E_n + R1_n Dt_{n-1} + R2_n Dt_{n-2},
//   E_n     = diag(beta) (V_n - e^{c_{n-1} + c_{n-2}} diag(e^gam) K_n S_{n-2}^T),
//
// with R1, R2 the state-independent 64 x 64 matrices the prep kernel stores (WsLag).
// The serial chain from one chunk's deltas to the next is then three small products
// (R2 Dt, R1 Dt, T E) in one wave, and everything that needs the state runs with a
// chunk of slack.  One workgroup per (seq, head, 16 value rows), five waves, one
// workgroup barrier per phase; every wave's inputs in phase t were published in
// phase t - 1 (buffers alternate by parity):
//   C  phase t:      Delta_t from E_t, Dt_{t-1}, Dt_{t-2}; publishes Delta_t, Dt_t
//   G  phase t:      E_{t+1} from S_{max(t-1,0)} (K_{t+1} rows, V_{t+1}, gates)
//   U  phase t >= 1: S_t = e^{c_{t-1}} S_{t-1} + K_{t-1}^T Dt_{t-1} (S^T in fp32
//                    accumulators, K^T from transposing LDS reads); publishes S_t;
//                    the final state after the last chunk
//   O  phase t >= 1: output rows of chunk t-1 from S_{t-1}, Delta_{t-1}, Q, P
//   P                K, V and gates moves into LDS rings (LDS-DMA)
// for t = -1 .. n_chunks.  C, G and O load their chunk operands two phases ahead
// straight into MFMA operand registers (fragment blocks and key/query rows, 16 bytes
// per lane; two register sets, so the kernel runs one workgroup per compute unit).
// The LDS-DMA moves are kept in a wave that reads no LDS: a wave with such moves in
// flight is made to wait for all of them before any LDS read of its own.
template <int D>
struct LagScan {
    static constexpr int KS = D / 32;        // 32-wide k steps over the key channels
    static constexpr int KT = D / 16;        // 16-key tiles of S^T
    static constexpr int NRB = D / 16;       // value tiles (workgroups) per (seq, head)
    static constexpr int RK = 2 * D + 32;    // K row stride in LDS: 2 mod 4 16-byte units
    static_assert((RK / 16) % 4 == 2, "K row stride");
    static constexpr int RV = 2 * 16 + 16;   // V row stride (the tile's 16 values)
    static constexpr int SK = 2, SV = 3;     // ring slots
    static constexpr int SG = 5;             // gates slots: chunk m is read in phases m-1 .. m+1
    static constexpr int kPubS = 0;                       // S^T: KS B-operand blocks, x 2
    static constexpr int kPubE = kPubS + 2 * KS * 1024;   // E: two B fragments, x 2
    static constexpr int kPubD = kPubE + 2 * 2048;        // Delta
    static constexpr int kPubDs = kPubD + 2 * 2048;       // Dt
    static constexpr int kK = kPubDs + 2 * 2048;
    static constexpr int kV = kK + SK * C * RK;
    static constexpr int kGt = kV + SV * C * RV;           // gates blocks (2 KiB each)
    static constexpr int kBytes = kGt + SG * 2048;
    static constexpr int NBK = C * RK / 1024;             // DMA blocks of one K slot
    static constexpr int NBV = C * RV / 1024;
    static constexpr int NBG = 2;
    static_assert(C * RK % 1024 == 0 && C * RV % 1024 == 0, "DMA blocks");
    static_assert(NBK + 2 * (NBV + NBG) < 64, "vmcnt range");
    static_assert(WsLag::kBytes - WsLag::kGates == 2048, "gates block");
};

struct LagPtrs {
    const unsigned char *k, *q;   // token 0 of (seq, key head)
    const unsigned char *v;       // token 0 of (seq, head), the tile's first value
    const unsigned char *ws;      // chunk 0 of (seq, head) in the workspace
    int64_t kq_bytes, hd_bytes;   // token strides of k/q and of v/out
    int64_t n_tokens;
    int nc;
    __device__ int nv(int m) const { return static_cast<int>(min<int64_t>(C, n_tokens - int64_t(m) * C)); }
    __device__ const unsigned char *wsc(int m) const { return ws + int64_t(m) * WsLag::kBytes; }
};

// Workgroup barrier of the lag scan: waits for this wave's LDS accesses only (the
// LDS-DMA loads in flight write slots nobody reads before their issuer has waited
// for them), and keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lag_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Keeps the compiler from moving memory accesses across this point: a wave issues
// its next chunk's operand loads only after this chunk's products have read the
// registers they replace (hoisting them would keep two sets of operands live).
__device__ __forceinline__ void lag_order() { asm volatile("" ::: "memory"); }

// Rows 16 tt + (lane mod 16) of a token-major matrix as A operands (k = 8g .. 8g + 7
// of each 32-wide step), rows at or past nv repeating row nv - 1.
template <int D>
__device__ __forceinline__ void load_row_frags(Frag<true> (&f)[4][D / 32], const unsigned char *base,
                                               int64_t stride, int nv, int lane)
{
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const unsigned char *p = base + int64_t(min(16 * tt + r, nv - 1)) * stride + 16 * g;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) f[tt][ks] = *reinterpret_cast<const Frag<true> *>(p + 64 * ks);
    }
}

// Gates row `row` of chunk m in the LDS ring.
template <int D>
__device__ __forceinline__ const float *lag_gates(const unsigned char *smem, int m, int row)
{
    return reinterpret_cast<const float *>(smem + LagScan<D>::kGt + (m % LagScan<D>::SG) * 2048) + row * C;
}

// Four gate values of the accumulator rows 16 tt + 4g .. 4g + 3 of one gates row.
__device__ __forceinline__ floatx4 gate4(const float *row, int tt, int lane)
{
    const float4 x = *reinterpret_cast<const float4 *>(row + 16 * tt + 4 * (lane >> 4));
    return floatx4{x.x, x.y, x.z, x.w};
}

// ---- C: the chain ----
struct LagCOps {
    Frag<true> ta[6], r1[8], r2[8];
};

__device__ __forceinline__ void lag_c_load(LagCOps &o, const LagPtrs &pp, int m, int lane)
{
    const unsigned char *wc = pp.wsc(m);
#pragma unroll
    for (int b = 0; b < 6; ++b) o.ta[b] = frag_blk<true>(wc + WsLag::kT + b * WsLag::kBlk, lane);
    if (m >= 1) {
#pragma unroll
        for (int b = 0; b < 8; ++b) o.r1[b] = frag_blk<true>(wc + WsLag::kR1 + b * WsLag::kBlk, lane);
    }
    if (m >= 2) {
#pragma unroll
        for (int b = 0; b < 8; ++b) o.r2[b] = frag_blk<true>(wc + WsLag::kR2 + b * WsLag::kBlk, lane);
    }
}

// The phase loops of C, G and O run two phases per iteration so that the operands
// of chunk m and m + 1 sit in two fixed register sets: the loads of chunk m + 2
// replace chunk m's set right after its products, two phases before use.
template <int D>
__device__ void lag_role_c(const LagPtrs &pp, unsigned char *smem, int lane, const LagTrace &tr)
{
    using F = LagScan<D>;
    const int nc = pp.nc;
    LagCOps oa, ob;
    Frag<true> dt1[2], dt2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        dt1[i].u = make_uint4(0u, 0u, 0u, 0u);
        dt2[i].u = make_uint4(0u, 0u, 0u, 0u);
    }
    lag_c_load(oa, pp, 0, lane);
    if (1 < nc) lag_c_load(ob, pp, 1, lane);
    auto step = [&](int t, LagCOps &o) {
        tr.mark(t, 0, lane);
        if (t >= 0 && t < nc) {
            tr.landed(t, lane);
            floatx4 acc[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) acc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (t >= 2) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    acc[tt] = mma(o.r2[2 * tt + 1], dt2[1], mma(o.r2[2 * tt], dt2[0], acc[tt]));
            }
            if (t >= 1) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    acc[tt] = mma(o.r1[2 * tt + 1], dt1[1], mma(o.r1[2 * tt], dt1[0], acc[tt]));
            }
            const Frag<true> *pe = reinterpret_cast<const Frag<true> *>(smem + F::kPubE + (t & 1) * 2048);
            tri_mul<true>(o.ta, pe[lane], pe[64 + lane], acc);
            // Dt = diag(e^{c - gam} (/|k|)) Delta
            const float *ed = lag_gates<D>(smem, t, 2);
            floatx4 ds[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) ds[tt] = gate4(ed, tt, lane) * acc[tt];
            Frag<true> *pd = reinterpret_cast<Frag<true> *>(smem + F::kPubD + (t & 1) * 2048);
            Frag<true> *ps = reinterpret_cast<Frag<true> *>(smem + F::kPubDs + (t & 1) * 2048);
            pd[lane] = acc_frag<true>(acc[0], acc[1]);
            pd[64 + lane] = acc_frag<true>(acc[2], acc[3]);
            dt2[0] = dt1[0];
            dt2[1] = dt1[1];
            dt1[0] = acc_frag<true>(ds[0], ds[1]);
            dt1[1] = acc_frag<true>(ds[2], ds[3]);
            ps[lane] = dt1[0];
            ps[64 + lane] = dt1[1];
            lag_order();   // the next operands replace this chunk's, not join them
            if (t + 2 < nc) lag_c_load(o, pp, t + 2, lane);
        }
        tr.mark(t, 2, lane);
        lag_barrier();
    };
    lag_barrier();                      // prologue
    // chunk m's operands are in oa for even m, ob for odd m
    for (int t = -1; t <= nc; t += 2) {
        step(t, ob);
        if (t + 1 <= nc) step(t + 1, oa);
    }
}

// ---- G: E one chunk ahead of the chain ----
template <int D>
struct LagGOps {
    Frag<true> gk[4][D / 32];      // K rows of the chunk
};

template <int D>
__device__ __forceinline__ void lag_g_load(LagGOps<D> &o, const LagPtrs &pp, int m, int lane)
{
    load_row_frags<D>(o.gk, pp.k + int64_t(m) * C * pp.kq_bytes, pp.kq_bytes, pp.nv(m), lane);
}

template <int D>
__device__ __forceinline__ void lag_g_dma_v(const LagPtrs &pp, unsigned char *smem, int m, int lane)
{
    using F = LagScan<D>;
    const uint32_t hdb = static_cast<uint32_t>(pp.hd_bytes);
    const unsigned char *vb = pp.v + int64_t(m) * C * pp.hd_bytes;
    unsigned char *slot = smem + F::kV + (m % F::SV) * C * F::RV;
#pragma unroll
    for (int i = 0; i < F::NBV; ++i)
        dma16(vb, dma_src_offset(i, lane, 16 * 2, F::RV, hdb, pp.nv(m)), slot + 1024 * i);
}

template <int D>
__device__ void lag_role_g(const LagPtrs &pp, unsigned char *smem, int lane, const LagTrace &tr)
{
    using F = LagScan<D>;
    const int nc = pp.nc;
    LagGOps<D> oa, ob;
    lag_g_load<D>(oa, pp, 0, lane);
    if (1 < nc) lag_g_load<D>(ob, pp, 1, lane);
    auto step = [&](int t, LagGOps<D> &o) {
        tr.mark(t, 0, lane);
        if (t <= nc - 2) {
            const int m = t + 1;        // chunk whose E is formed
            tr.landed(t, lane);
            const int src = t - 1 > 0 ? t - 1 : 0;   // S_{max(m-2, 0)}
            Frag<true> bs[F::KS];
#pragma unroll
            for (int ks = 0; ks < F::KS; ++ks)
                bs[ks] = frag_blk<true>(smem + F::kPubS + ((src & 1) * F::KS + ks) * 1024, lane);
            floatx4 x[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                x[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < F::KS; ++ks) x[tt] = mma(o.gk[tt][ks], bs[ks], x[tt]);
            }
            const unsigned char *vs = smem + F::kV + (m % F::SV) * C * F::RV;
            // e^{c_{m-1} + c_{m-2}} (fewer factors for the first chunks)
            const float f = (m >= 1 ? lag_gates<D>(smem, m - 1, 3)[0] : 1.f) *
                            (m >= 2 ? lag_gates<D>(smem, m - 2, 3)[0] : 1.f);
            const float *gb = lag_gates<D>(smem, m, 0), *ge = lag_gates<D>(smem, m, 1);
            floatx4 e[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const floatx4 vv = col4<true>(vs, F::RV, 16 * tt, 0, lane);
                const floatx4 b4 = gate4(gb, tt, lane), e4 = gate4(ge, tt, lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) e[tt][j] = b4[j] * fmaf(-f * e4[j], x[tt][j], vv[j]);
            }
            Frag<true> *pe = reinterpret_cast<Frag<true> *>(smem + F::kPubE + (m & 1) * 2048);
            pe[lane] = acc_frag<true>(e[0], e[1]);
            pe[64 + lane] = acc_frag<true>(e[2], e[3]);
            lag_order();
            if (m + 2 < nc) lag_g_load<D>(o, pp, m + 2, lane);
        }
        tr.mark(t, 2, lane);
        lag_barrier();
    };
    lag_barrier();                      // prologue
    // phase t forms E of chunk t + 1: even chunks in oa, odd in ob
    for (int t = -1; t <= nc; t += 2) {
        step(t, oa);
        if (t + 1 <= nc) step(t + 1, ob);
    }
}

// ---- U: the state pass ----
template <int D>
__device__ __forceinline__ void lag_publish_s(const floatx4 (&Mt)[D / 16], unsigned char *blocks, int lane)
{
    const int gq = lane >> 4, cl = lane & 15;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
        // keys 16t + 4gq + 0..3: block t/2, unit group 2 (t & 1) + gq / 2, elements 4 (gq & 1) ..
        unsigned char *u = blocks + (t >> 1) * 1024 + 16 * blk_unit(cl, 2 * (t & 1) + (gq >> 1)) +
                           8 * (gq & 1);
        *reinterpret_cast<uint2 *>(u) = make_uint2(pack2(Mt[t][0], Mt[t][1]), pack2(Mt[t][2], Mt[t][3]));
    }
}

template <int D>
__device__ __forceinline__ void lag_u_dma_k(const LagPtrs &pp, unsigned char *smem, int m, int lane)
{
    using F = LagScan<D>;
    const unsigned char *kb = pp.k + int64_t(m) * C * pp.kq_bytes;
    unsigned char *slot = smem + F::kK + (m % F::SK) * C * F::RK;
    const uint32_t kqb = static_cast<uint32_t>(pp.kq_bytes);
#pragma unroll
    for (int i = 0; i < F::NBK; ++i)
        dma16(kb, dma_src_offset(i, lane, 2 * D, F::RK, kqb, pp.nv(m)), slot + 1024 * i);
}

template <int D>
__device__ void lag_role_u(const LagPtrs &pp, unsigned char *smem, const float *state_in,
                           float *state_out, int64_t st_off, int lane, const LagTrace &tr)
{
    using F = LagScan<D>;
    const int nc = pp.nc;
    floatx4 Mt[F::KT];
#pragma unroll
    for (int t = 0; t < F::KT; ++t) {
        if (state_in) {
            const float4 m = *reinterpret_cast<const float4 *>(state_in + st_off + 16 * t);
            Mt[t] = floatx4{m.x, m.y, m.z, m.w};
        } else {
            Mt[t] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }
    lag_publish_s<D>(Mt, smem + F::kPubS, lane);
    Frag<true> akt[F::KT][2];
    lag_barrier();                      // prologue
    for (int t = -1; t <= nc; ++t) {
        tr.mark(t, 0, lane);
        if (t >= 1) {
            const Frag<true> *ps = reinterpret_cast<const Frag<true> *>(smem + F::kPubDs + ((t - 1) & 1) * 2048);
            const Frag<true> d0 = ps[lane], d1 = ps[64 + lane];
            const float ec = lag_gates<D>(smem, t - 1, 3)[0];
#pragma unroll
            for (int kt = 0; kt < F::KT; ++kt) Mt[kt] *= ec;
#pragma unroll
            for (int kt = 0; kt < F::KT; ++kt) Mt[kt] = mma(akt[kt][0], d0, Mt[kt]);
#pragma unroll
            for (int kt = 0; kt < F::KT; ++kt) Mt[kt] = mma(akt[kt][1], d1, Mt[kt]);
            lag_publish_s<D>(Mt, smem + F::kPubS + (t & 1) * F::KS * 1024, lane);
        }
        if (t >= 0 && t < nc) {
            // K_t was moved in by P before this phase began
            tr.mark(t, 1, lane);
            const unsigned char *kslot = smem + F::kK + (t % F::SK) * C * F::RK;
#pragma unroll
            for (int kt = 0; kt < F::KT; ++kt) {
                akt[kt][0] = frag_cols<true>(kslot, F::RK, 0, 16 * kt, lane);
                akt[kt][1] = frag_cols<true>(kslot, F::RK, 32, 16 * kt, lane);
            }
        }
        tr.mark(t, 2, lane);
        lag_barrier();
    }
#pragma unroll
    for (int t = 0; t < F::KT; ++t)
        *reinterpret_cast<float4 *>(state_out + st_off + 16 * t) =
            make_float4(Mt[t][0], Mt[t][1], Mt[t][2], Mt[t][3]);
}

// ---- P: K and V moves into LDS ----
// Phase t moves K_{t+1} (U reads it at the end of phase t+1; two slots, the rows
// are in L2 already, G having loaded them in phase t-1), V_{t+3} (G reads it in
// phase t+2; three slots) and the gates block of chunk t+3 (read by G, C, U and O
// in phases t+2 .. t+4; five slots), then waits for K_{t+1}, which with the issue
// order also covers chunk t+2's moves: every move is complete before the barrier
// after which it is read.
// P reads no LDS itself, so no wait on its moves is forced anywhere else.
template <int D>
__device__ __forceinline__ void lag_p_dma_vg(const LagPtrs &pp, unsigned char *smem, int m, int lane)
{
    using F = LagScan<D>;
    lag_g_dma_v<D>(pp, smem, m, lane);
    const unsigned char *gb = pp.wsc(m) + WsLag::kGates;
    unsigned char *slot = smem + F::kGt + (m % F::SG) * 2048;
#pragma unroll
    for (int i = 0; i < F::NBG; ++i) dma16(gb, 1024u * i + 16u * lane, slot + 1024 * i);
}

template <int D>
__device__ void lag_role_p(const LagPtrs &pp, unsigned char *smem, int lane)
{
    const int nc = pp.nc;
    constexpr int NVG = LagScan<D>::NBV + LagScan<D>::NBG;
    lag_p_dma_vg<D>(pp, smem, 0, lane);
    if (1 < nc) lag_p_dma_vg<D>(pp, smem, 1, lane);
    if (1 < nc) wait_vmem_le<NVG>(); else wait_vmem_le<0>();   // V_0, gates_0 (phase -1)
    lag_barrier();                      // prologue
    for (int t = -1; t <= nc; ++t) {
        if (t + 1 < nc) lag_u_dma_k<D>(pp, smem, t + 1, lane);
        if (t + 3 < nc) lag_p_dma_vg<D>(pp, smem, t + 3, lane);
        if (t + 3 < nc) wait_vmem_le<NVG>(); else wait_vmem_le<0>();
        lag_barrier();
    }
}

// ---- O: the output ----
template <int D>
struct LagOOps {
    Frag<true> oq[4][D / 32];      // Q rows
    Frag<true> op[6];              // P / sqrt(d) blocks
};

template <int D>
__device__ __forceinline__ void lag_o_load(LagOOps<D> &o, const LagPtrs &pp, int m, int lane)
{
    load_row_frags<D>(o.oq, pp.q + int64_t(m) * C * pp.kq_bytes, pp.kq_bytes, pp.nv(m), lane);
    const unsigned char *wc = pp.wsc(m);
#pragma unroll
    for (int b = 0; b < 6; ++b) o.op[b] = frag_blk<true>(wc + WsLag::kP + b * WsLag::kBlk, lane);
}

template <int D>
__device__ void lag_role_o(const LagPtrs &pp, unsigned char *smem, uint16_t *obase, int lane,
                           const LagTrace &tr)
{
    using F = LagScan<D>;
    const int nc = pp.nc;
    const int gq = lane >> 4, cl = lane & 15;
    const int64_t hd = pp.hd_bytes / 2;
    LagOOps<D> oa, ob;
    lag_o_load<D>(oa, pp, 0, lane);
    if (1 < nc) lag_o_load<D>(ob, pp, 1, lane);
    auto step = [&](int t, LagOOps<D> &o) {
        tr.mark(t, 0, lane);
        if (t >= 1) {
            tr.landed(t, lane);
            const int m = t - 1;        // chunk whose rows are written
            Frag<true> bm[F::KS];
#pragma unroll
            for (int ks = 0; ks < F::KS; ++ks)
                bm[ks] = frag_blk<true>(smem + F::kPubS + ((m & 1) * F::KS + ks) * 1024, lane);
            const float *eg = lag_gates<D>(smem, m, 4);   // e^gam (/|q|)
            floatx4 acc[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                floatx4 xq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < F::KS; ++ks) xq = mma(bm[ks], o.oq[tt][ks], xq);
                acc[tt] = xq * (kOutScale<D> * eg[16 * tt + cl]);
            }
            const Frag<true> *pd = reinterpret_cast<const Frag<true> *>(smem + F::kPubD + (m & 1) * 2048);
            const Frag<true> d0 = pd[lane], d1 = pd[64 + lane];
            acc[0] = mma(d0, o.op[0], acc[0]);
            acc[1] = mma(d0, o.op[1], acc[1]);
            acc[2] = mma(d1, o.op[3], mma(d0, o.op[2], acc[2]));
            acc[3] = mma(d1, o.op[5], mma(d0, o.op[4], acc[3]));
            // the next operand loads go out before the stores: loads issued after them
            // could be given the stores' data registers and would wait for the stores
            lag_order();
            if (m + 2 < nc) lag_o_load<D>(o, pp, m + 2, lane);
            uint16_t *ob_ = obase + int64_t(m) * C * hd;
            const int nv = pp.nv(m);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                if (nv == C || 16 * tt + cl < nv)
                    *reinterpret_cast<uint2 *>(ob_ + (16 * tt + cl) * hd + 4 * gq) =
                        make_uint2(pack2(acc[tt][0], acc[tt][1]), pack2(acc[tt][2], acc[tt][3]));
            }
        }
        tr.mark(t, 2, lane);
        lag_barrier();
    };
    lag_barrier();                      // prologue
    // phase t writes chunk t - 1: even chunks in oa, odd in ob
    for (int t = -1; t <= nc; t += 2) {
        step(t, oa);
        if (t + 1 <= nc) step(t + 1, ob);
    }
}

// Workgroups are numbered so that the NRB row blocks of one (seq, head) share the
// low three bits of the block id and land on one XCD (shared L2).
constexpr int kLagWaves = 5;

// Two register sets of operands per wave (up to 256 registers): one workgroup per
// compute unit.
template <int D>
__global__ __launch_bounds__(64 * kLagWaves) __attribute__((amdgpu_waves_per_eu(2))) void chunk_lag_kernel(
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *state_in, void *__restrict__ out, float *state_out,
    const unsigned char *__restrict__ ws, int64_t n_tokens, int64_t n_heads, int64_t n_k_heads,
    int64_t n_sh, int n_chunks)
{
    using F = LagScan<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    const int64_t b = blockIdx.x;
    const int64_t sh = (b / (8 * F::NRB)) * 8 + (b & 7);
    const int rb = static_cast<int>((b >> 3) % F::NRB);
    if (sh >= n_sh) return;   // whole workgroup leaves before any barrier
    const int64_t s = sh / n_heads, h = sh - s * n_heads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int v0 = 16 * rb;
    LagPtrs pp;
    pp.kq_bytes = n_k_heads * D * 2;
    pp.hd_bytes = n_heads * D * 2;
    const int64_t ktok0 = (s * n_tokens * n_k_heads + h % n_k_heads) * D;
    const int64_t tok0 = (s * n_tokens * n_heads + h) * D;
    pp.k = static_cast<const unsigned char *>(k) + ktok0 * 2;
    pp.q = static_cast<const unsigned char *>(q) + ktok0 * 2;
    pp.v = static_cast<const unsigned char *>(v) + (tok0 + v0) * 2;
    pp.ws = ws + sh * n_chunks * WsLag::kBytes;
    pp.n_tokens = n_tokens;
    pp.nc = n_chunks;
    const LagTrace tr{static_cast<int>(b), wave};
    if (wave == 0) {
        lag_role_c<D>(pp, smem, lane, tr);
    } else if (wave == 1) {
        lag_role_g<D>(pp, smem, lane, tr);
    } else if (wave == 2) {
        const int64_t st_off = sh * D * D + int64_t(v0 + (lane & 15)) * D + 4 * (lane >> 4);
        lag_role_u<D>(pp, smem, state_in, state_out, st_off, lane, tr);
    } else if (wave == 3) {
        lag_role_o<D>(pp, smem, static_cast<uint16_t *>(out) + tok0 + v0, lane, tr);
    } else {
        lag_role_p<D>(pp, smem, lane);
    }
}

template <int D>
int64_t lag_blocks(int64_t n_sh)
{
    return (n_sh + 7) / 8 * 8 * LagScan<D>::NRB;
}

// The lag scan: one workgroup per compute unit (its registers allow no second one;
// the LDS request says so as well).
template <int D>
hipError_t launch_lag(const Problem &p, const unsigned char *ws, int n_chunks, hipStream_t stream)
{
    using F = LagScan<D>;
    constexpr int kAlone = 80 * 1024 + 256;
    static_assert(F::kBytes <= kAlone, "LDS of the lag scan");
    auto kern = chunk_lag_kernel<D>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = ensure_lds_limit(kern, kAlone, lds_set);
    if (e != hipSuccess) return e;
    const int64_t blocks = lag_blocks<D>(p.n_seqs * p.n_heads);
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(64 * kLagWaves), kAlone,
                       stream, p.q, p.k, p.v, p.state_in, p.out, p.state_out, ws, p.n_tokens,
                       p.n_heads, p.n_k_heads, p.n_seqs * p.n_heads, n_chunks);
    return hipGetLastError();
}

}  // namespace

bool lag_pass_fits(int64_t n_sh, int head_dim)
{
    switch (head_dim) {
    case 32: return grid_fits(lag_blocks<32>(n_sh), 64 * kLagWaves);
    case 64: return grid_fits(lag_blocks<64>(n_sh), 64 * kLagWaves);
    case 96: return grid_fits(lag_blocks<96>(n_sh), 64 * kLagWaves);
    case 128: return grid_fits(lag_blocks<128>(n_sh), 64 * kLagWaves);
    default: return false;
    }
}

hipError_t launch_lag_pass(const Problem &p, const unsigned char *ws, int n_chunks,
                           hipStream_t stream)
{
    switch (p.head_dim) {
    case 32: return launch_lag<32>(p, ws, n_chunks, stream);
    case 64: return launch_lag<64>(p, ws, n_chunks, stream);
    case 96: return launch_lag<96>(p, ws, n_chunks, stream);
    case 128: return launch_lag<128>(p, ws, n_chunks, stream);
    default: return hipErrorInvalidValue;
    }
}

#ifdef GDN_PHASE_TRACE
// Copies the phase timestamps of the last lag pass out (trace builds only; not part
// of the installed interface).
extern "C" int gdn_phase_trace_read(void *host, size_t bytes)
{
    if (bytes > sizeof(g_phase_trace)) bytes = sizeof(g_phase_trace);
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_trace), bytes, 0, hipMemcpyDeviceToHost) ==
                   hipSuccess
               ? 0
               : -1;
}
#endif

}  // namespace gdn
