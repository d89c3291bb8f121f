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
    int64_t q_sb, q_sh, q_ss;
    int64_t k_sb, k_sw;
    int64_t w_sb, w_ss;
    int32_t B, S, H, D, W, m;
    int32_t n_chunks;  // row chunks of kBwdChunkRows rows
    int32_t n_jtiles;  // key tiles of kBwdKeyTile entries
    float scale;
};

// Rows of one chunk of the key-gradient pass; each (chunk, key tile) pair
// writes one partial that a reduction sums in chunk order.
constexpr int kBwdChunkRows = 256;
// Entries of one key tile of the key-gradient pass (4 waves x 32 entries).
constexpr int kBwdKeyTile = 128;

// Bytes of partials csa_index_score_backward needs for this shape.
inline size_t bwd_workspace_bytes(int B, int S, int W, int D)
{
    size_t chunks = ((size_t)S + kBwdChunkRows - 1) / kBwdChunkRows;
    return (size_t)B * chunks * (size_t)W * (size_t)D * sizeof(float);
}

// Each returns hipSuccess or the launch error; nothing is synchronised.
// dq and dw (one pass over the key tiles per block of query rows).
hipError_t launch_bwd_rows(int D, int HB, const BwdArgs &a, hipStream_t s);
// Per-chunk partial key gradients (one pass over the rows per key tile).
hipError_t launch_bwd_keys(int D, int HB, const BwdArgs &a, hipStream_t s);
// dk = scale * sum over live chunks of the partials.
hipError_t launch_bwd_reduce(const BwdArgs &a, hipStream_t s);

} // namespace csa
