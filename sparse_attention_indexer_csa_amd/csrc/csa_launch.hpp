// Launch interface between the C ABI (csa_api.cpp) and the kernels
// (csa_kernels.hip).  Host-side only declarations plus the argument block
// the kernels receive by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

struct KernelArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *w;
    const int32_t *q_offset;
    const int32_t *q_seg;
    const int32_t *k_seg;
    float *scores;   // [rows, W] (rows = B*S), dense
    int32_t *idx;    // [rows, top_k]
    const float *target; // KL mode: [rows, W] target weights (>= 0), dense
    float *kl;           // KL mode: [rows] divergence of each row
    int64_t q_sb, q_sh, q_ss;
    int64_t k_sb, k_sw;
    int64_t w_sb, w_ss;
    int64_t rows;    // B*S (top-k kernel: number of rows)
    int32_t B, S, H, W, m;
    int32_t top_k, cap;
    int32_t n_row_blocks; // row-tile plan: ceil(S / rows per workgroup)
    int32_t n_chunks;     // split plan: workgroups per row
    int32_t full_rows;    // split plan: write every score of the row (-inf past the visible prefix)
    int32_t limit_rows;   // top-k kernel: rows end at their visible prefix (q_offset, m)
    int32_t redo;         // top-k kernels in two passes: see kTopkRedo
    float scale;
};

// Row-tile plan geometry.
constexpr int kRowWaves = 4;            // waves per workgroup, one query row each
constexpr int kRowsPerBlock = kRowWaves;
constexpr int kTileEntries = 64;        // compressed entries per LDS K tile
// Split plan geometry.
constexpr int kSplitWaves = 4;
constexpr int kSplitTiles = 4;          // 64-entry tiles per wave
constexpr int kSplitChunk = kSplitWaves * kSplitTiles * kTileEntries;
// Balanced split plan: rows it takes, one workgroup of eight waves per
// compute unit.  (With two four-wave workgroups per compute unit the older
// one won the issue arbitration throughout, and the younger one's equal
// share of the tiles ended up to 20 us later.)
constexpr int kStreamRows = 256;
constexpr int kStreamWaves = 8;
constexpr int kStreamBlocksPerCU = 1;
// Top-k kernel geometry: one wave per row, or one workgroup per long row.
constexpr int kTopkWaves = 4;
constexpr int kTopkBlockWaves = 8;
// Rows at least this long use the workgroup-per-row top-k.
constexpr int kTopkBlockMinLen = 8192;

enum { kModeScores = 1, kModeSelect = 2, kModeKL = 4 };
// Added by the row-tile launcher when the call has document segments, so the
// kernels without them carry no segment code.
constexpr int kModeSegs = 8;

// Candidate-buffer capacity of the streaming top-k for a given k (room for at
// least one more 64-pair push after a compaction down to k).  The row-tile
// kernel stores 16-bit entries and affords a larger buffer, so most rows never
// compact mid-stream.
__host__ __device__ constexpr int topk_capacity(int k) { return ((k + 63) / 64) * 64 + 512; }
// With up to two head blocks the row-tile kernel runs three workgroups per
// compute unit and its buffers are smaller.
__host__ __device__ constexpr int rows_topk_capacity(int k, int HB)
{
    return ((k + 63) / 64) * 64 + (HB <= 2 ? 704 : 1024);
}
// LDS bytes of one wave's row-tile buffer: histogram, keys, 16-bit entries,
// each array with 64 slots past cap.
__host__ __device__ constexpr size_t rows_topk_wave_bytes(int cap) { return 1024 + (size_t)(cap + 64) * 6; }
// Entries of the row-tile plan are stored in 16 bits.
constexpr int kRowTilesMaxW = 65536;

size_t rows_lds_bytes(int D, int HB, int mode, int cap);
size_t topk_lds_bytes(int cap);
size_t topk_block_lds_bytes(int cap, int top_k, int W);
// LDS of the workgroup-per-row kernel without its streaming fallback (the
// in-LDS path alone), or 0 when that path cannot take rows of W entries or
// would rarely succeed for k (k above 1920).
size_t topk_block_fast_only_lds_bytes(int top_k, int W);
// Two-pass top-k, for k whose streaming fallback does not fit in one
// workgroup's LDS: with redo set, topk_block_kernel writes a row that its
// in-LDS path cannot take as kTopkRedo in the row's first output, and
// topk_kernel then selects only the rows so marked.
constexpr int32_t kTopkRedo = -2;

// Each returns hipSuccess or the launch error; nothing is synchronised.
hipError_t launch_rows(int D, int HB, int mode, const KernelArgs &a, size_t lds, hipStream_t s);
hipError_t launch_split(int D, int HB, const KernelArgs &a, hipStream_t s);
// Balanced split over `blocks` workgroups; rows <= kStreamRows, scores of the
// visible prefixes only.
hipError_t launch_stream(int D, int HB, const KernelArgs &a, int blocks, hipStream_t s);
hipError_t launch_topk(const KernelArgs &a, size_t lds, hipStream_t s);
hipError_t launch_topk_block(const KernelArgs &a, size_t lds, hipStream_t s);
// KL divergence and its gradient from a dense score matrix held in a.scores
// (-inf where masked): a.kl gets each row's divergence, a.scores is
// overwritten with d kl / d score.
hipError_t launch_kl_grad(const KernelArgs &a, hipStream_t s);

} // namespace csa
