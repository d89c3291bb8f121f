// Launch interface of the backward kernels (csa_backward.hip): gradients of
// the indexer score with respect to q, k and w.  Host-side declarations plus
// the argument block the kernels receive by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

struct BwdArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *w;
    const int32_t *q_offset;
    const int32_t *q_seg;
    const int32_t *k_seg;
    const float *g;  // [B,S,W] upstream gradient of the scores, dense
    float *dq;       // [B,H,S,D] dense
    float *dk;       // [B,W,D] dense
    float *dw;       // [B,S,H] dense
    float *part;     // [B, n_chunks, W, D] per-row-chunk partial key gradients
    uint32_t *sign;  // [B, S, n_blk, H] logit signs: bit e of word (b,i,jb,h) is [l > 0] of
                     // entry 32jb + entry_of_bit(e), written by the row pass, read by the key pass
    int64_t q_sb, q_sh, q_ss;
    int64_t k_sb, k_sw;
    int64_t w_sb, w_ss;
    int32_t B, S, H, D, W, m;
    int32_t n_chunks;  // row chunks of kBwdChunkRows rows
    int32_t n_jtiles;  // key tiles of kBwdKeyTile entries
    int32_t n_blk;     // 32-entry blocks: ceil(W / 32)
    float scale;
};

// Rows of one chunk of the key-gradient pass; each (chunk, key tile) pair
// writes one partial that a reduction sums in chunk order.
constexpr int kBwdChunkRows = 256;
// Entries of one key tile of the key-gradient pass (4 waves x 32 entries).
constexpr int kBwdKeyTile = 128;

// Workspace of csa_index_score_backward: the partials, then (256-byte
// aligned) the logit-sign words.
inline size_t bwd_partials_bytes(int B, int S, int W, int D)
{
    size_t chunks = ((size_t)S + kBwdChunkRows - 1) / kBwdChunkRows;
    return (size_t)B * chunks * (size_t)W * (size_t)D * sizeof(float);
}

inline size_t bwd_sign_offset(int B, int S, int W, int D)
{
    return (bwd_partials_bytes(B, S, W, D) + 255) / 256 * 256;
}

inline size_t bwd_workspace_bytes(int B, int S, int W, int D, int H)
{
    const size_t blocks = ((size_t)W + 31) / 32;
    const size_t sign = (size_t)B * (size_t)S * blocks * (size_t)H * sizeof(uint32_t);
    return sign ? bwd_sign_offset(B, S, W, D) + sign : bwd_partials_bytes(B, S, W, D);
}

// Each returns hipSuccess or the launch error; nothing is synchronised.
// dq and dw (one pass over the key tiles per block of query rows).
hipError_t launch_bwd_rows(int D, int HB, const BwdArgs &a, hipStream_t s);
// Per-chunk partial key gradients (one pass over the rows per key tile).
hipError_t launch_bwd_keys(int D, int HB, const BwdArgs &a, hipStream_t s);
// dk = scale * sum over live chunks of the partials.
hipError_t launch_bwd_reduce(const BwdArgs &a, hipStream_t s);

} // namespace csa
