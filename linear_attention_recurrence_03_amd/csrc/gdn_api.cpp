// gdn_api.cpp -- the C-ABI of libgdn: host-side validation and dispatch.
//
// Every check runs before any HIP call, so that a rejected call launches
// nothing (and so that the checks can be exercised on a machine without a
// GPU).  The contract is documented in include/gdn.h.
#include "gdn.h"

#include <limits.h>
#include <stdint.h>

#include <cmath>

#include "gdn_internal.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

// Largest element count accepted for one tensor: far beyond any device memory,
// small enough that every byte offset fits comfortably in int64.
constexpr int64_t kMaxElems = int64_t(1) << 40;

// A dispatch counts the work-items of its grid in 32 bits, so one call is bounded
// by the grids it launches: state rows (n_seqs * n_heads * head_dim; the token
// recurrence runs 8 work-items per row, the chunked scan at most 28) and, for the
// chunked form, chunks (n_seqs * n_heads * ceil(n_tokens / 64); 256 work-items
// each).  Both bounds lie beyond what fits in device memory at head_dim 128.
constexpr int64_t kMaxStateRows = int64_t(1) << 27;
constexpr int64_t kMaxChunks = (int64_t(1) << 24) - 1;
constexpr int64_t kMaxChunkRowsBytes = int64_t(1) << 32;

bool mul_ok(int64_t a, int64_t b, int64_t *r)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > kMaxElems / a) return false;
    *r = a * b;
    return *r <= kMaxElems;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void *p, int64_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b)
{
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// AUTO: the chunked form from the length at which it overtakes the token recurrence
// on MI355X (one sequence, 8 or 32 heads, d=128, device time per call): bf16 at 16
// tokens (10.4 vs 10.2 us; 14.1 vs 10.2 at 24), fp32 at 40 (16.3 vs 17.9 us at 32,
// 22.6 vs 18.0 at 48; the fp32 chunked path keeps one ring slot).
// AUTO: the chunked form from the token count at which it overtakes the token
// recurrence on MI355X. The recurrence costs a fixed latency per token while few
// state rows are in flight and ALU time proportional to the rows once they fill
// the chip, so the crossover falls as the work per token grows; the work is
// counted in d = 128 heads (n_seqs * n_heads * (d / 128)^2, measured at d = 128).
gdn_algo pick_algo(gdn_algo algo, int64_t n_seqs, int64_t n_tokens, int64_t n_heads,
                   int head_dim, gdn_dtype dtype)
{
    if (algo != GDN_ALGO_AUTO) return algo;
    const double units = static_cast<double>(n_seqs) * static_cast<double>(n_heads) *
                         (head_dim / 128.0) * (head_dim / 128.0);
    int64_t from;
    if (dtype == GDN_BF16)
        from = units <= 96 ? 20 : units <= 192 ? 18 : units <= 512 ? 16 : 14;
    else   // the fp32 chunked form runs fp32 MFMA, a step per 64 tokens: a later crossover
        from = units <= 40 ? 48 : units <= 96 ? 60 : units <= 192 ? 104 : 120;
    return n_tokens >= from ? GDN_ALGO_CHUNKED : GDN_ALGO_RECURRENT;
}

bool is_chunked(gdn_algo a)
{
    return a == GDN_ALGO_CHUNKED || a == GDN_ALGO_CHUNKED_LAG || a == GDN_ALGO_CHUNKED_HEAD;
}

// Shape checks shared by gdn_workspace_size and gdn_forward.  On success fills
// the element counts of a token tensor, a gate tensor and the state.
int check_shape(gdn_dtype dtype, int64_t n_seqs, int64_t n_tokens, int64_t n_heads,
                int head_dim, gdn_algo algo, int64_t *tok_elems, int64_t *gate_elems,
                int64_t *state_elems)
{
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
    if (algo != GDN_ALGO_AUTO && algo != GDN_ALGO_RECURRENT && algo != GDN_ALGO_CHUNKED &&
        algo != GDN_ALGO_CHUNKED_LAG && algo != GDN_ALGO_CHUNKED_HEAD)
        return GDN_ERR_ALGO_UNAVAILABLE;
    if ((algo == GDN_ALGO_CHUNKED_LAG || algo == GDN_ALGO_CHUNKED_HEAD) && dtype != GDN_BF16)
        return GDN_ERR_ALGO_UNAVAILABLE;
    if (!gdn_supports(head_dim)) return GDN_ERR_UNSUPPORTED_HEAD_DIM;
    if (n_seqs < 0 || n_tokens < 0 || n_heads < 0) return GDN_ERR_BAD_SHAPE;
    int64_t a, b;
    if (!mul_ok(n_seqs, n_tokens, &a) || !mul_ok(a, n_heads, gate_elems) ||
        !mul_ok(*gate_elems, head_dim, tok_elems))
        return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(n_seqs, n_heads, &b) || !mul_ok(b, int64_t(head_dim) * head_dim, state_elems))
        return GDN_ERR_BAD_SHAPE;
    if (b * head_dim > kMaxStateRows) return GDN_ERR_BAD_SHAPE;
    if (b > 0 && n_tokens > 0 &&
        is_chunked(pick_algo(algo, n_seqs, n_tokens, n_heads, head_dim, dtype))) {
        if ((n_tokens + 63) / 64 > kMaxChunks / b) return GDN_ERR_BAD_SHAPE;
        // The chunked kernels form the byte offset of a token row inside one chunk
        // of q, k or v in 32 bits: 64 token rows of every head must span < 4 GiB.
        const int64_t esz = (dtype == GDN_BF16) ? 2 : 4;
        if (64 * n_heads * head_dim * esz >= kMaxChunkRowsBytes) return GDN_ERR_BAD_SHAPE;
    }
    return GDN_OK;
}

// Element counts of the decode-attention tensors.
struct AttnSizes {
    int64_t q_elems, kv_elems, mask_elems, out_elems;
};

// Shape checks of the decode attention (sizes may be null).
int attn_check(int64_t n_seqs, int64_t n_heads, int64_t n_heads_kv, int64_t n_q, int64_t n_kv,
               int head_dim, float scale, AttnSizes *sizes)
{
    if (!(head_dim == 64 || head_dim == 128 || head_dim == 256)) return GDN_ERR_UNSUPPORTED_HEAD_DIM;
    if (n_seqs < 0 || n_heads < 0 || n_heads_kv < 0 || n_kv < 0) return GDN_ERR_BAD_SHAPE;
    if (n_q < 1 || n_q >= 20) return GDN_ERR_BAD_SHAPE;
    if (!std::isfinite(scale)) return GDN_ERR_BAD_SHAPE;
    if (n_heads > 0 && (n_heads_kv == 0 || n_heads % n_heads_kv != 0)) return GDN_ERR_BAD_SHAPE;
    int64_t a, b, c, d;
    if (!mul_ok(n_seqs, n_heads, &a) || !mul_ok(a, n_q, &b) || !mul_ok(b, head_dim, &c))
        return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(n_seqs, n_heads_kv, &a) || !mul_ok(a, n_kv, &b) || !mul_ok(b, head_dim, &d))
        return GDN_ERR_BAD_SHAPE;
    int64_t m;
    if (!mul_ok(n_seqs, n_q, &a) || !mul_ok(a, n_kv, &m)) return GDN_ERR_BAD_SHAPE;
    // grids: (seq, key/value head, row group, token range) workgroups of 256
    // work-items, then one wave per (seq, query, head) row to merge the ranges; a
    // dispatch counts work-items in 32 bits
    if (n_seqs * n_heads * n_q > (int64_t(1) << 24)) return GDN_ERR_BAD_SHAPE;
    // the kernels index cache positions in 32 bits
    if (n_kv >= (int64_t(1) << 31)) return GDN_ERR_BAD_SHAPE;
    if (n_seqs > 0 && n_heads > 0 && !gdn::attn_grid_fits(n_seqs, n_heads, n_heads_kv, n_q, n_kv))
        return GDN_ERR_BAD_SHAPE;
    if (sizes) {
        sizes->q_elems = c;
        sizes->out_elems = c;
        sizes->kv_elems = d;
        sizes->mask_elems = m;
    }
    return GDN_OK;
}

// gdn_forward with n_key_heads query/key heads (value head h reads key head
// h % n_key_heads); gdn_forward is the case n_key_heads == n_heads.
int forward_impl(gdn_dtype dtype, const void *q, const void *k, const void *v, const float *g,
                 const float *beta, const float *state_in, void *out, float *state_out,
                 int64_t n_seqs, int64_t n_tokens, int64_t n_heads, int64_t n_key_heads,
                 int head_dim, unsigned flags, void *workspace, size_t workspace_bytes,
                 gdn_algo algo, void *stream, bool use_scratch = false);

}  // namespace

extern "C" {

int gdn_supports(int head_dim)
{
    return (head_dim >= 32 && head_dim <= 128 && head_dim % 32 == 0) ? 1 : 0;
}

size_t gdn_workspace_size(gdn_dtype dtype, int64_t n_seqs, int64_t n_tokens,
                          int64_t n_heads, int head_dim, gdn_algo algo)
{
    int64_t te, ge, se;
    if (check_shape(dtype, n_seqs, n_tokens, n_heads, head_dim, algo, &te, &ge, &se) != GDN_OK)
        return 0;
    if (n_seqs == 0 || n_heads == 0 || n_tokens == 0) return 0;
    const gdn_algo chosen = pick_algo(algo, n_seqs, n_tokens, n_heads, head_dim, dtype);
    if (!is_chunked(chosen)) return 0;
    return gdn::chunk_workspace_bytes(dtype == GDN_BF16, chosen == GDN_ALGO_CHUNKED_LAG, n_seqs,
                                      n_tokens, n_heads, head_dim);
}

int gdn_forward(gdn_dtype dtype, const void *q, const void *k, const void *v, const float *g,
                const float *beta, const float *state_in, void *out, float *state_out,
                int64_t n_seqs, int64_t n_tokens, int64_t n_heads, int head_dim,
                void *workspace, size_t workspace_bytes, gdn_algo algo, void *stream)
{
    return forward_impl(dtype, q, k, v, g, beta, state_in, out, state_out, n_seqs, n_tokens,
                        n_heads, n_heads, head_dim, GDN_PRE_NONE, workspace, workspace_bytes,
                        algo, stream);
}

int gdn_forward_tiled(gdn_dtype dtype, const void *q, const void *k, const void *v,
                      const float *g, const float *beta, const float *state_in, void *out,
                      float *state_out, int64_t n_seqs, int64_t n_tokens, int64_t n_heads,
                      int64_t n_key_heads, int head_dim, void *workspace,
                      size_t workspace_bytes, gdn_algo algo, void *stream)
{
    return forward_impl(dtype, q, k, v, g, beta, state_in, out, state_out, n_seqs, n_tokens,
                        n_heads, n_key_heads, head_dim, GDN_PRE_NONE, workspace,
                        workspace_bytes, algo, stream);
}

int gdn_forward_ex(gdn_dtype dtype, const void *q, const void *k, const void *v, const float *g,
                   const float *beta, const float *state_in, void *out, float *state_out,
                   int64_t n_seqs, int64_t n_tokens, int64_t n_heads, int64_t n_key_heads,
                   int head_dim, unsigned int flags, void *workspace, size_t workspace_bytes,
                   gdn_algo algo, void *stream)
{
    return forward_impl(dtype, q, k, v, g, beta, state_in, out, state_out, n_seqs, n_tokens,
                        n_heads, n_key_heads, head_dim, flags, workspace, workspace_bytes, algo,
                        stream);
}

int gdn_forward_noalloc(gdn_dtype dtype, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, const float *state_in, void *out,
                        float *state_out, int64_t n_seqs, int64_t n_tokens, int64_t n_heads,
                        int64_t n_key_heads, int head_dim, unsigned int flags, gdn_algo algo,
                        void *stream)
{
    // forward_impl validates everything first (a call needing more than the scratch
    // array is refused there) and looks the array up only once the call is valid
    return forward_impl(dtype, q, k, v, g, beta, state_in, out, state_out, n_seqs, n_tokens,
                        n_heads, n_key_heads, head_dim, flags, nullptr,
                        gdn::kNoAllocScratchBytes, algo, stream, true);
}

size_t gdn_noalloc_scratch_bytes(void)
{
    return gdn::kNoAllocScratchBytes;
}

int gdn_flash_attn_supports(int n_q, int head_dim_k, int head_dim_v)
{
    const bool width = head_dim_k == head_dim_v &&
                       (head_dim_k == 64 || head_dim_k == 128 || head_dim_k == 256);
    return (n_q >= 1 && n_q < 20 && width) ? 1 : 0;
}

size_t gdn_flash_attn_workspace_size(int64_t n_seqs, int64_t n_heads, int64_t n_heads_kv,
                                     int64_t n_q, int64_t n_kv, int head_dim)
{
    if (attn_check(n_seqs, n_heads, n_heads_kv, n_q, n_kv, head_dim, 1.f, nullptr) != GDN_OK)
        return 0;
    if (n_seqs == 0 || n_heads == 0) return 0;
    return gdn::attn_workspace_bytes(n_seqs, n_heads, n_heads_kv, n_q, n_kv, head_dim);
}

int gdn_flash_attn(gdn_dtype dtype, const void *q, const void *k, const void *v,
                   const float *mask, void *out, int64_t n_seqs, int64_t n_heads,
                   int64_t n_heads_kv, int64_t n_q, int64_t n_kv, int head_dim, float scale,
                   void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
    AttnSizes z;
    int rc = attn_check(n_seqs, n_heads, n_heads_kv, n_q, n_kv, head_dim, scale, &z);
    if (rc != GDN_OK) return rc;
    if (n_seqs == 0 || n_heads == 0) return GDN_OK;
    const int64_t esz = (dtype == GDN_BF16) ? 2 : 4;
    if (!q || !out) return GDN_ERR_NULL_POINTER;
    if (n_kv > 0 && (!k || !v)) return GDN_ERR_NULL_POINTER;
    const void *ptrs[] = {q, k, v, mask, out, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_MISALIGNED;
    const Range r_out = range_of(out, z.out_elems * esz);
    const Range reads[] = {range_of(q, z.q_elems * esz), range_of(k, z.kv_elems * esz),
                           range_of(v, z.kv_elems * esz),
                           mask ? range_of(mask, z.mask_elems * 4) : Range{0, 0}};
    for (const Range &r : reads)
        if (overlap(r_out, r)) return GDN_ERR_ALIASING;
    const size_t need = gdn::attn_workspace_bytes(n_seqs, n_heads, n_heads_kv, n_q, n_kv,
                                                  head_dim);
    if (workspace_bytes < need) return GDN_ERR_WORKSPACE_TOO_SMALL;
    if (need > 0) {
        if (!workspace) return GDN_ERR_NULL_POINTER;
        const Range r_ws = range_of(workspace, static_cast<int64_t>(need));
        for (const Range &r : reads)
            if (overlap(r_ws, r)) return GDN_ERR_ALIASING;
        if (overlap(r_ws, r_out)) return GDN_ERR_ALIASING;
    }

    // ---- validated: from here on only launches ----
    gdn::AttnProblem p;
    p.bf16 = (dtype == GDN_BF16);
    p.q = q;
    p.k = k;
    p.v = v;
    p.mask = mask;
    p.out = out;
    p.scale = scale;
    p.n_seqs = n_seqs;
    p.n_heads = n_heads;
    p.n_heads_kv = n_heads_kv;
    p.n_q = n_q;
    p.n_kv = n_kv;
    p.head_dim = head_dim;
    const hipError_t err = gdn::launch_attn(p, workspace, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

const char *gdn_status_string(int status)
{
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head_dim (need 32, 64, 96 or 128)";
    case GDN_ERR_BAD_SHAPE: return "bad shape (negative or too large size)";
    case GDN_ERR_NULL_POINTER: return "required pointer is NULL";
    case GDN_ERR_BAD_DTYPE: return "bad dtype (need GDN_F32 or GDN_BF16)";
    case GDN_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than gdn_workspace_size()";
    case GDN_ERR_ALGO_UNAVAILABLE: return "algorithm value not recognised, or not available for the dtype";
    case GDN_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case GDN_ERR_ALIASING: return "output overlaps an input (only state_out == state_in is allowed)";
    case GDN_ERR_HIP: return "HIP runtime refused a launch";
    case GDN_ERR_BAD_FLAGS: return "unknown bits in the input-transform flags";
    case GDN_ERR_SCRATCH_TOO_SMALL:
        return "gdn_forward_noalloc: the call needs more scratch than the library's fixed "
               "array (gdn_noalloc_scratch_bytes()); use gdn_forward_ex with a workspace";
    default: return "unknown status";
    }
}

int gdn_version(void)
{
    return kVersion;
}

}  // extern "C"

namespace {

int forward_impl(gdn_dtype dtype, const void *q, const void *k, const void *v, const float *g,
                 const float *beta, const float *state_in, void *out, float *state_out,
                 int64_t n_seqs, int64_t n_tokens, int64_t n_heads, int64_t n_key_heads,
                 int head_dim, unsigned flags, void *workspace, size_t workspace_bytes,
                 gdn_algo algo, void *stream, bool use_scratch)
{
    int64_t tok_elems, gate_elems, state_elems;
    int rc = check_shape(dtype, n_seqs, n_tokens, n_heads, head_dim, algo, &tok_elems,
                         &gate_elems, &state_elems);
    if (rc != GDN_OK) return rc;
    if (flags & ~unsigned(GDN_PRE_L2NORM_QK | GDN_PRE_RAW_GATES)) return GDN_ERR_BAD_FLAGS;
    if (n_key_heads < 0) return GDN_ERR_BAD_SHAPE;
    if (n_heads > 0 && (n_key_heads == 0 || n_heads % n_key_heads != 0)) return GDN_ERR_BAD_SHAPE;
    if (n_seqs == 0 || n_heads == 0) return GDN_OK;
    // elements of q and k (n_key_heads heads; at most those of v)
    const int64_t kq_elems = tok_elems / n_heads * n_key_heads;

    const int64_t esz = (dtype == GDN_BF16) ? 2 : 4;
    const bool have_tokens = n_tokens > 0;
    if (!state_out) return GDN_ERR_NULL_POINTER;
    if (have_tokens && (!q || !k || !v || !g || !beta || !out)) return GDN_ERR_NULL_POINTER;

    const void *ptrs[] = {q, k, v, g, beta, state_in, out, state_out, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_MISALIGNED;

    const Range r_state_out = range_of(state_out, state_elems * 4);
    const Range r_state_in = state_in ? range_of(state_in, state_elems * 4) : Range{0, 0};
    if (state_in && state_in != state_out && overlap(r_state_in, r_state_out))
        return GDN_ERR_ALIASING;
    if (have_tokens) {
        const Range r_out = range_of(out, tok_elems * esz);
        const Range reads[] = {range_of(q, kq_elems * esz), range_of(k, kq_elems * esz),
                               range_of(v, tok_elems * esz), range_of(g, gate_elems * 4),
                               range_of(beta, gate_elems * 4)};
        for (const Range &r : reads)
            if (overlap(r_out, r) || overlap(r_state_out, r)) return GDN_ERR_ALIASING;
        if (overlap(r_out, r_state_in) || overlap(r_out, r_state_out)) return GDN_ERR_ALIASING;
    }

    const gdn_algo chosen = pick_algo(algo, n_seqs, n_tokens, n_heads, head_dim, dtype);
    size_t need = 0;
    if (have_tokens && is_chunked(chosen)) {
        need = gdn::chunk_workspace_bytes(dtype == GDN_BF16, chosen == GDN_ALGO_CHUNKED_LAG,
                                          n_seqs, n_tokens, n_heads, head_dim);
        if (use_scratch) {
            // gdn_forward_noalloc: the library's fixed array, looked up only now that
            // the call is known to be valid and to fit (the first HIP call of the entry)
            if (need > workspace_bytes) return GDN_ERR_SCRATCH_TOO_SMALL;
            if (gdn::noalloc_scratch(&workspace) != hipSuccess) return GDN_ERR_HIP;
        }
        if (workspace_bytes < need) return GDN_ERR_WORKSPACE_TOO_SMALL;
        if (need > 0 && !workspace) return GDN_ERR_NULL_POINTER;
        if (need > 0) {
            const Range r_ws = range_of(workspace, static_cast<int64_t>(need));
            const Range all[] = {range_of(q, kq_elems * esz), range_of(k, kq_elems * esz),
                                 range_of(v, tok_elems * esz), range_of(g, gate_elems * 4),
                                 range_of(beta, gate_elems * 4), r_state_in, r_state_out,
                                 range_of(out, tok_elems * esz)};
            for (const Range &r : all)
                if (overlap(r_ws, r)) return GDN_ERR_ALIASING;
        }
    }

    // ---- validated: from here on only launches ----
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (!have_tokens) {
        if (state_in == state_out) return GDN_OK;
        err = gdn::launch_state_copy(state_in, state_out, state_elems, st);
        return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    }
    gdn::Problem p;
    p.bf16 = (dtype == GDN_BF16);
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.state_in = state_in;
    p.out = out;
    p.state_out = state_out;
    p.n_seqs = n_seqs;
    p.n_tokens = n_tokens;
    p.n_heads = n_heads;
    p.n_k_heads = n_key_heads;
    p.l2norm_qk = (flags & GDN_PRE_L2NORM_QK) ? 1 : 0;
    p.raw_gates = (flags & GDN_PRE_RAW_GATES) ? 1 : 0;
    p.head_dim = head_dim;
    // AUTO picks the chunk-to-chunk pass by grid size; the forced values keep theirs
    p.head_scan = algo == GDN_ALGO_CHUNKED_HEAD ? 1 : algo == GDN_ALGO_CHUNKED ? -1 : 0;
    if (is_chunked(chosen))
        err = gdn::launch_chunked(p, chosen == GDN_ALGO_CHUNKED_LAG, workspace, st);
    else
        err = gdn::launch_recurrent(p, st);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace

