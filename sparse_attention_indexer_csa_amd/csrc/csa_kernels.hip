// gfx950 kernels of the CSA indexer: the row-tile score / fused select
// kernel, the split-row score kernel for long rows, and the row top-k kernel.
#include <math.h>

#include "csa_device.hpp"
#include "csa_launch.hpp"
#include "csa_score.hpp"
#include "csa_topk.hpp"

namespace csa {

template <int D>
struct TileGeom {
    static constexpr int kKs = D / 32;                      // MFMA k-steps per entry
    static constexpr int kPitch = D + 8;                    // LDS row pitch (elements): +16 B
    static constexpr int kChunks = kTileEntries * D / 8;    // 16-byte pieces per tile
    static constexpr int kPerThread = kChunks / (kRowWaves * kWave);
    static constexpr size_t kTileBytes = (size_t)kTileEntries * kPitch * 2;
};

// ---------------------------------------------------------------------------
// Row-tile plan.  A workgroup owns kRowsPerBlock consecutive query rows of one
// batch row (one row per wave) and walks the compressed keys in tiles of
// kTileEntries entries staged in LDS and shared by its waves.  Tiles past the
// last row's visible prefix are never loaded.  Workgroups are issued from the
// longest rows (largest i) down so that the causal tail finishes early.
//
// mode & kModeScores: every score of the rows is written (masked = -inf).
// mode & kModeSelect: each wave streams its row's scores through a TopKRow
//                     candidate buffer in LDS and writes the row's top-k.
// ---------------------------------------------------------------------------
template <int D, int HB, int MODE>
__global__ __launch_bounds__(kRowWaves * kWave) void rows_kernel(const KernelArgs a)
{
    using G = TileGeom<D>;
    constexpr int KS = G::kKs;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t *ktile = reinterpret_cast<uint16_t *>(smem);

    const int tid = threadIdx.x;
    const int wv = tid / kWave;
    const int l = lane();

    const int rb = a.n_row_blocks - 1 - (int)(blockIdx.x / a.B);
    const int b = (int)(blockIdx.x % a.B);
    const int row0 = rb * kRowsPerBlock;
    const int i = row0 + wv;
    const bool active = i < a.S;

    const int64_t off = a.q_offset ? (int64_t)a.q_offset[b] : 0;
    const int last = min(row0 + kRowsPerBlock, a.S) - 1;
    const int thr_last = visible_entries(off + last, a.m, a.W);
    const int ntiles = (thr_last + kTileEntries - 1) / kTileEntries;
    const int thr = active ? visible_entries(off + i, a.m, a.W) : 0;
    const int qseg = (a.q_seg && active) ? a.q_seg[(int64_t)b * a.S + i] : 0;
    const int32_t *kseg = a.k_seg ? a.k_seg + (int64_t)b * a.W : nullptr;
    const int64_t row_id = (int64_t)b * a.S + i;

    RowOperand<HB, KS> row;
    if (active)
        load_row<HB, KS>(row, a.q + b * a.q_sb + (int64_t)i * a.q_ss, a.q_sh, a.w + b * a.w_sb + (int64_t)i * a.w_ss,
                         a.H);

    TopKRow tk;
    if (MODE & kModeSelect) {
        unsigned char *base = smem + G::kTileBytes + (size_t)wv * (1024 + (size_t)a.cap * 8);
        uint32_t *hist = reinterpret_cast<uint32_t *>(base);
        uint32_t *key = hist + 256;
        topk_init(tk, key, key + a.cap, hist, a.cap, a.top_k);
    }

    const uint16_t *kb = a.k + b * a.k_sb;
    u32x4 pre[G::kPerThread];
    auto fetch = [&](int t) {
#pragma unroll
        for (int x = 0; x < G::kPerThread; ++x) {
            const int c = tid + x * kRowWaves * kWave;
            const int e = c / (D / 8), p = c % (D / 8);
            const int j = t * kTileEntries + e;
            pre[x] = (j < a.W) ? *reinterpret_cast<const u32x4 *>(kb + (int64_t)j * a.k_sw + p * 8)
                               : u32x4{0u, 0u, 0u, 0u};
        }
    };
    if (ntiles > 0)
        fetch(0);

    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();
#pragma unroll
        for (int x = 0; x < G::kPerThread; ++x) {
            const int c = tid + x * kRowWaves * kWave;
            const int e = c / (D / 8), p = c % (D / 8);
            *reinterpret_cast<u32x4 *>(ktile + e * G::kPitch + p * 8) = pre[x];
        }
        __syncthreads();
        if (t + 1 < ntiles)
            fetch(t + 1);

        if (!active)
            continue;
        const int j0 = t * kTileEntries;
        float sv = -INFINITY;
        if (j0 < thr) {
#pragma unroll
            for (int st = 0; st < kTileEntries / 16; ++st) {
                const int js = j0 + st * 16;
                if (js < thr) {
                    bool any = true;
                    if (kseg) {
                        const int jj = js + (l & 15);
                        any = ballot(jj < thr && kseg[jj] == qseg) != 0ull;
                    }
                    if (any) {
                        bf16x8 bf[KS];
                        load_entries_lds<KS>(bf, ktile, st * 16, G::kPitch);
                        const float s = scaled_score(subtile_score<HB, KS>(row, bf), a.scale);
                        if ((l >> 4) == st)
                            sv = s;
                    }
                }
            }
        }
        const int j = j0 + l;
        bool valid = j < thr;
        if (valid && kseg)
            valid = kseg[j] == qseg;
        const float outv = valid ? sv : -INFINITY;
        if (MODE & kModeScores) {
            if (j < a.W)
                a.scores[row_id * a.W + j] = outv;
        }
        if (MODE & kModeSelect)
            topk_push(tk, score_key(outv), (uint32_t)j, valid);
    }

    if (!active)
        return;
    if (MODE & kModeScores) {
        for (int j = ntiles * kTileEntries + l; j < a.W; j += kWave)
            a.scores[row_id * a.W + j] = -INFINITY;
    }
    if (MODE & kModeSelect)
        topk_finish(tk, a.idx + row_id * a.top_k);
}

// ---------------------------------------------------------------------------
// Split-row plan (long rows, few of them: decode).  Workgroup (row, chunk)
// scores kSplitChunk consecutive entries of one row; each wave takes
// kSplitSubtiles subtiles and reads its keys straight from HBM (every key byte
// is used by one row only, so there is nothing to share through LDS).  Only
// the visible prefix of the row is read.  Scores go to a.scores with row
// stride W; with full_rows the rest of the row is filled with -inf.
// ---------------------------------------------------------------------------
template <int D, int HB>
__global__ __launch_bounds__(kSplitWaves * kWave) void split_kernel(const KernelArgs a)
{
    constexpr int KS = D / 32;
    constexpr int kWaveEntries = kSplitSubtiles * 16;
    const int wv = threadIdx.x / kWave;
    const int l = lane();
    const int64_t row_id = blockIdx.x / a.n_chunks;
    const int chunk = (int)(blockIdx.x % a.n_chunks);
    const int b = (int)(row_id / a.S), i = (int)(row_id % a.S);
    const int64_t off = a.q_offset ? (int64_t)a.q_offset[b] : 0;
    const int thr = visible_entries(off + i, a.m, a.W);
    const int base = chunk * kSplitChunk + wv * kWaveEntries;
    float *out = a.scores + row_id * a.W;

    if (base >= thr) {
        if (a.full_rows)
            for (int j = base + l; j < min(base + kWaveEntries, a.W); j += kWave)
                out[j] = -INFINITY;
        return;
    }
    const int qseg = a.q_seg ? a.q_seg[row_id] : 0;
    const int32_t *kseg = a.k_seg ? a.k_seg + (int64_t)b * a.W : nullptr;

    RowOperand<HB, KS> row;
    load_row<HB, KS>(row, a.q + b * a.q_sb + (int64_t)i * a.q_ss, a.q_sh, a.w + b * a.w_sb + (int64_t)i * a.w_ss, a.H);
    const uint16_t *kb = a.k + b * a.k_sb;

#pragma unroll 1
    for (int g4 = 0; g4 < kSplitSubtiles / 4; ++g4) {
        const int j0 = base + g4 * 64;
        if (j0 >= thr && !a.full_rows)
            break;
        float sv = -INFINITY;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int js = j0 + st * 16;
            if (js < thr) {
                bool any = true;
                if (kseg) {
                    const int jj = js + (l & 15);
                    any = ballot(jj < thr && kseg[jj] == qseg) != 0ull;
                }
                if (any) {
                    bf16x8 bf[KS];
                    load_entries_global<KS>(bf, kb, a.k_sw, js, thr);
                    const float s = scaled_score(subtile_score<HB, KS>(row, bf), a.scale);
                    if ((l >> 4) == st)
                        sv = s;
                }
            }
        }
        const int j = j0 + l;
        bool valid = j < thr;
        if (valid && kseg)
            valid = kseg[j] == qseg;
        if (j < a.W && (a.full_rows || j < thr))
            out[j] = valid ? sv : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Row top-k over a dense fp32 score matrix: one wave per row streams the row
// through a TopKRow buffer.  With limit_rows the row ends at its visible
// prefix (used after the split plan, whose rows are only written that far).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kTopkWaves * kWave) void topk_kernel(const KernelArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int wv = threadIdx.x / kWave;
    const int l = lane();
    const int64_t row = (int64_t)blockIdx.x * kTopkWaves + wv;
    if (row >= a.rows)
        return;
    int n = a.W;
    if (a.limit_rows) {
        const int b = (int)(row / a.S), i = (int)(row % a.S);
        const int64_t off = a.q_offset ? (int64_t)a.q_offset[b] : 0;
        n = visible_entries(off + i, a.m, a.W);
    }
    unsigned char *base = smem + (size_t)wv * (1024 + (size_t)a.cap * 8);
    uint32_t *hist = reinterpret_cast<uint32_t *>(base);
    uint32_t *key = hist + 256;
    TopKRow tk;
    topk_init(tk, key, key + a.cap, hist, a.cap, a.top_k);
    const float *src = a.scores + row * a.W;
#pragma unroll 1
    for (int j0 = 0; j0 < n; j0 += kWave) {
        const int j = j0 + l;
        const float s = (j < n) ? src[j] : -INFINITY;
        const uint32_t kv = score_key(s);
        topk_push(tk, kv, (uint32_t)j, j < n && key_selectable(kv));
    }
    topk_finish(tk, a.idx + row * a.top_k);
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------
size_t rows_lds_bytes(int D, int mode, int cap)
{
    size_t tile = (size_t)kTileEntries * (D + 8) * 2;
    size_t sel = (mode & kModeSelect) ? (size_t)kRowWaves * (1024 + (size_t)cap * 8) : 0;
    return tile + sel;
}

size_t topk_lds_bytes(int cap) { return (size_t)kTopkWaves * (1024 + (size_t)cap * 8); }

template <typename K>
static hipError_t launch(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, const KernelArgs &a)
{
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(kernel, grid, block, lds, s, a);
    return hipGetLastError();
}

template <int D, int HB>
static hipError_t launch_rows_t(int mode, const KernelArgs &a, size_t lds, hipStream_t s)
{
    dim3 grid((unsigned)((int64_t)a.B * a.n_row_blocks)), block(kRowWaves * kWave);
    switch (mode) {
    case kModeScores:
        return launch(rows_kernel<D, HB, kModeScores>, grid, block, lds, s, a);
    case kModeSelect:
        return launch(rows_kernel<D, HB, kModeSelect>, grid, block, lds, s, a);
    case kModeScores | kModeSelect:
        return launch(rows_kernel<D, HB, kModeScores | kModeSelect>, grid, block, lds, s, a);
    default:
        return hipErrorInvalidValue;
    }
}

template <int D>
static hipError_t launch_rows_d(int HB, int mode, const KernelArgs &a, size_t lds, hipStream_t s)
{
    switch (HB) {
    case 1: return launch_rows_t<D, 1>(mode, a, lds, s);
    case 2: return launch_rows_t<D, 2>(mode, a, lds, s);
    case 4: return launch_rows_t<D, 4>(mode, a, lds, s);
    case 8: return launch_rows_t<D, 8>(mode, a, lds, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rows(int D, int HB, int mode, const KernelArgs &a, size_t lds, hipStream_t s)
{
    switch (D) {
    case 32: return launch_rows_d<32>(HB, mode, a, lds, s);
    case 64: return launch_rows_d<64>(HB, mode, a, lds, s);
    case 128: return launch_rows_d<128>(HB, mode, a, lds, s);
    default: return hipErrorInvalidValue;
    }
}

template <int D>
static hipError_t launch_split_d(int HB, const KernelArgs &a, hipStream_t s)
{
    dim3 grid((unsigned)(a.rows * a.n_chunks)), block(kSplitWaves * kWave);
    switch (HB) {
    case 1: return launch(split_kernel<D, 1>, grid, block, 0, s, a);
    case 2: return launch(split_kernel<D, 2>, grid, block, 0, s, a);
    case 4: return launch(split_kernel<D, 4>, grid, block, 0, s, a);
    case 8: return launch(split_kernel<D, 8>, grid, block, 0, s, a);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_split(int D, int HB, const KernelArgs &a, hipStream_t s)
{
    switch (D) {
    case 32: return launch_split_d<32>(HB, a, s);
    case 64: return launch_split_d<64>(HB, a, s);
    case 128: return launch_split_d<128>(HB, a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_topk(const KernelArgs &a, size_t lds, hipStream_t s)
{
    dim3 grid((unsigned)((a.rows + kTopkWaves - 1) / kTopkWaves)), block(kTopkWaves * kWave);
    return launch(topk_kernel, grid, block, lds, s, a);
}

} // namespace csa
