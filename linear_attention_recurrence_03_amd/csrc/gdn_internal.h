// gdn_internal.h -- launchers shared between the C-ABI layer and the kernels.
// Not installed; the public interface is include/gdn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Chunk length of the chunked algorithm (tokens per block of the sequence).
constexpr int kChunk = 64;

// A dispatch counts the work-items of its grid in 32 bits.
inline bool grid_fits(int64_t blocks, int64_t threads)
{
    return blocks > 0 && threads > 0 && blocks <= int64_t(0xffffffffLL) / threads;
}

struct Problem {
    int bf16;               // 1: q, k, v, out are bf16; 0: fp32
    const void *q, *k, *v;
    const float *g, *beta;
    const float *state_in;  // may be null (zero initial state)
    void *out;
    float *state_out;
    int64_t n_seqs, n_tokens, n_heads;
    int64_t n_k_heads;      // heads of q and k; value head h reads head h % n_k_heads
    int head_dim;
    int l2norm_qk;          // 1: q and k rows are divided by sqrt(|row|^2 + 1e-6)
    int raw_gates;          // 1: g <- -softplus(g), beta <- sigmoid(beta)
    int head_scan = 0;      // chunked bf16: 1 whole-head pass, -1 per-tile pass, 0 by size
};

// Token recurrence, any n_tokens >= 1.
hipError_t launch_recurrent(const Problem &p, hipStream_t stream);

// Chunked algorithm, n_tokens >= 1.  Needs chunk_workspace_bytes(...) bytes.  lag:
// the two-chunk-lag scan (bf16 rows only).
size_t chunk_workspace_bytes(int bf16, int lag, int64_t n_seqs, int64_t n_tokens,
                             int64_t n_heads, int head_dim);
hipError_t launch_chunked(const Problem &p, bool lag, void *workspace, hipStream_t stream);

// The chunk-to-chunk passes kept in files of their own (bf16 rows), run after the
// prep kernel has filled the workspace: the whole-head pass (gdn_chunk_head.hip) and
// the two-chunk-lag pass (gdn_chunk_lag.hip), with the grid checks done before any
// kernel of a call is launched.
bool head_pass_fits(int64_t n_sh, int head_dim);
hipError_t launch_head_pass(const Problem &p, const unsigned char *ws, int n_chunks,
                            hipStream_t stream);
bool lag_pass_fits(int64_t n_sh, int head_dim);
hipError_t launch_lag_pass(const Problem &p, const unsigned char *ws, int n_chunks,
                           hipStream_t stream);

// Size of the library-owned scratch array behind gdn_forward_noalloc (one per
// device), and its address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void **ptr);

// n_tokens == 0: state_out = state_in (or zeros when state_in is null).
hipError_t launch_state_copy(const float *state_in, float *state_out,
                             int64_t count, hipStream_t stream);

// ---- decode flash attention ----------------------------------------------------

struct AttnProblem {
    int bf16;               // 1: q, k, v, out are bf16; 0: fp32
    const void *q, *k, *v;  // q (S, H, n_q, D); k, v (S, Hkv, n_kv, D)
    const float *mask;      // (S, 1, n_q, n_kv) additive, or null
    void *out;              // (S, n_q, H, D)
    float scale;
    int64_t n_seqs, n_heads, n_heads_kv, n_q, n_kv;
    int head_dim;           // 64, 128 or 256
};

// How the cache is cut: rows of one (seq, key/value head) in groups of four, and
// n_split token ranges of split_len tokens.
struct AttnSplit {
    int groups, n_split, split_len;
};
AttnSplit attn_split(int64_t n_seqs, int64_t n_heads, int64_t n_heads_kv, int64_t n_q,
                     int64_t n_kv);
size_t attn_workspace_bytes(int64_t n_seqs, int64_t n_heads, int64_t n_heads_kv, int64_t n_q,
                            int64_t n_kv, int head_dim);
// Whether both attention grids fit one dispatch each (n_seqs, n_heads >= 1 and
// n_heads_kv a divisor of n_heads).
bool attn_grid_fits(int64_t n_seqs, int64_t n_heads, int64_t n_heads_kv, int64_t n_q,
                    int64_t n_kv);
hipError_t launch_attn(const AttnProblem &p, void *workspace, hipStream_t stream);

}  // namespace gdn
