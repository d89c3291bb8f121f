// gfx950 kernels of the CSA indexer: the row-tile score / fused select
// kernel, the split-row score kernel for long rows, and the row top-k kernels.
#include <math.h>

#include "csa_device.hpp"
#include "csa_launch.hpp"
#include "csa_score.hpp"
#include "csa_topk.hpp"

namespace csa {

// LDS image of a key tile: kTileEntries rows of D bf16 with a 16-byte pad
// per row (row pitch D+8 elements), so the 16-byte B-fragment reads of
// consecutive entries fall in different bank groups.  The tile is filled by
// buffer-to-LDS DMA: instruction x writes the 64 consecutive 16-byte slots
// 64x .. 64x+63 of the image, lane l the slot 64x+l; slot s holds chunk
// s % kRowChunks of entry s / kRowChunks (pad slots receive whatever follows
// the entry and are never read).  A tile is kRowChunks instructions.
template <int D>
struct TileGeom {
    static constexpr int kKs = D / 16;                      // MFMA k-steps per entry
    static constexpr int kPitch = D + 8;                    // LDS row pitch (elements): +16 B
    static constexpr int kRowChunks = kPitch / 8;           // 16-byte slots per LDS row
    static constexpr int kDmaOps = kRowChunks;              // 64 * kRowChunks slots / 64 lanes
    static constexpr int kDmaPerWave = (kDmaOps + kRowWaves - 1) / kRowWaves;
    static constexpr int kTileElems = kTileEntries * kPitch;
    static constexpr size_t kTileBytes = (size_t)kTileElems * 2;
};

// Buffer resource over `bytes` bytes at `base` (raw, 32-bit elements): loads
// at or beyond `bytes` return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// Bytes a buffer resource must cover for n consecutive entries of D bf16 at
// a stride of entry_bytes: from the first entry's start to the end of the
// last entry's D values.  Strides below the row width (overlapping entries,
// or 0 for a single entry) are covered as well as padded ones.  16-byte
// slots past that range (row pads) read zeros and are never consumed.
template <int D>
__device__ __forceinline__ int entries_span(int n, int entry_bytes)
{
    return n > 0 ? (n - 1) * entry_bytes + 2 * D : 0;
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voffset, 0, 0, 0);
}

// Waits for this wave's outstanding vector-memory operations (the tile DMA).
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Waits until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order), and for its LDS operations.
template <int N>
__device__ __forceinline__ void vm_wait_le()
{
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// First 64-entry unit u < nunits that holds an entry j < thr of segment qseg
// (nunits if there is none).  The segment ids of eight units are loaded at
// once, so a row whose segment starts late costs a few memory round trips,
// not one per unit.
__device__ __forceinline__ int first_segment_unit(const int32_t *kseg, int thr, int qseg, int nunits, int W)
{
    constexpr int kBatch = 8;
    const int l = lane();
    for (int u0 = 0; u0 < nunits; u0 += kBatch) {
        int v[kBatch];
#pragma unroll
        for (int r = 0; r < kBatch; ++r)
            v[r] = kseg[min((u0 + r) * kTileEntries + l, W - 1)];
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
            const int j = (u0 + r) * kTileEntries + l;
            if (u0 + r < nunits && ballot(j < thr && v[r] == qseg) != 0ull)
                return u0 + r;
        }
    }
    return nunits;
}

// Scores of the 64 entries j0 .. j0+63 of one row: lane l returns the
// scaled score of entry j0 + l.  Subtiles (32 entries) flagged off are not
// computed (their lanes return garbage that the caller masks).  `load(b, sub)`
// fills the B fragments of subtile sub.
template <int HB, int KS, typename LoadB>
__device__ __forceinline__ float tile_scores(const RowOperand<HB, KS> &row, bool do0, bool do1, float scale,
                                             LoadB load)
{
    float p0 = 0.0f, p1 = 0.0f;
    if (do0) {
        bf16x8 b[KS];
        load(b, 0);
        p0 = subtile_partial<HB, KS>(row, b);
    }
    if (do1) {
        bf16x8 b[KS];
        load(b, 1);
        p1 = subtile_partial<HB, KS>(row, b);
    }
    return scaled_score(combine_halves(p0, p1), scale);
}

// ---------------------------------------------------------------------------
// Indexer KL loss of one row, accumulated over its visible entries: a running
// maximum m and sum of exp(s - m) (an online log-sum-exp), the target mass A
// and C = sum of a (log a - s) over entries with target a > 0.  Then
//   KL = C / A + (m + log sum) - log A,
// which is sum of p (log p - s + lse) with p = a / A.  A lane holds the
// statistics of the entries it has seen; kl_merge combines two holders.
// ---------------------------------------------------------------------------
struct KLAcc {
    float m, se, A, C;
};

__device__ __forceinline__ KLAcc kl_empty() { return KLAcc{-INFINITY, 0.0f, 0.0f, 0.0f}; }

// One visible entry with finite score s and target weight a >= 0.
__device__ __forceinline__ void kl_add(KLAcc &k, float s, float a)
{
    const float mn = fmaxf(k.m, s);
    k.se = k.se * __expf(k.m - mn) + __expf(s - mn);
    k.m = mn;
    k.A += a;
    k.C += a > 0.0f ? a * (__logf(a) - s) : 0.0f;
}

__device__ __forceinline__ KLAcc kl_merge(const KLAcc &x, const KLAcc &y)
{
    const float mn = fmaxf(x.m, y.m);
    KLAcc r;
    r.m = mn;
    r.se = (mn == -INFINITY) ? 0.0f : x.se * __expf(x.m - mn) + y.se * __expf(y.m - mn);
    r.A = x.A + y.A;
    r.C = x.C + y.C;
    return r;
}

// Butterfly combine over the 64 lanes (every lane ends with the total).
__device__ __forceinline__ KLAcc kl_wave_reduce(KLAcc k)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        KLAcc o;
        o.m = __shfl_xor(k.m, off, kWave);
        o.se = __shfl_xor(k.se, off, kWave);
        o.A = __shfl_xor(k.A, off, kWave);
        o.C = __shfl_xor(k.C, off, kWave);
        // both partners combine (lower lane's statistics first) to the same bits
        k = (lane() & off) ? kl_merge(o, k) : kl_merge(k, o);
    }
    return k;
}

// The divergence from a row's totals: 0 without a visible entry or target mass.
__device__ __forceinline__ float kl_value(const KLAcc &k)
{
    if (k.m == -INFINITY || !(k.A > 0.0f))
        return 0.0f;
    return k.C / k.A + (k.m + __logf(k.se)) - __logf(k.A);
}

// ---------------------------------------------------------------------------
// Row-tile plan.  A workgroup owns kRowsPerBlock consecutive query rows of one
// batch row (one row per wave) and walks the compressed keys in tiles of
// kTileEntries entries, double-buffered in LDS and shared by its waves (one
// barrier per tile; the next tile's global loads are in flight during the
// current tile's MFMAs).  Tiles past the last row's visible prefix are never
// loaded.  Workgroups are issued from the longest rows (largest i) down so
// the causal tail finishes early.
//
// mode & kModeScores: every score of the rows is written (masked = -inf).
// mode & kModeSelect: each wave streams its row's scores through a TopKRow
//                     candidate buffer in LDS and writes the row's top-k.
// mode & kModeKL:     each wave folds its row's scores and target weights
//                     into KL statistics (KLAcc) and writes the row's
//                     divergence; the target of a tile is loaded one tile
//                     ahead of its use.
// ---------------------------------------------------------------------------
// This kernel serves rows of more than 64 heads (four head blocks), one wave
// per SIMD; up to 64 heads rows3_kernel below takes the plan.
template <int D, int HB, int MODE>
__global__ __launch_bounds__(kRowWaves * kWave) __attribute__((amdgpu_waves_per_eu(1)))
void rows_kernel(const KernelArgs a)
{
    using G = TileGeom<D>;
    constexpr int KS = G::kKs;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t *ktile = reinterpret_cast<uint16_t *>(smem);

    const int tid = threadIdx.x;
    const int wv = uniform(tid / kWave);
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

    // With segments, tiles before the first one that holds an entry of any
    // row's segment are masked for the whole workgroup and are skipped.
    int t_lo = 0;
    if (kseg) {
        __shared__ int first_tile[kRowWaves];
        const int ft = active ? first_segment_unit(kseg, thr, qseg, ntiles, a.W) : ntiles;
        if (l == 0)
            first_tile[wv] = ft;
        __syncthreads();
#pragma unroll
        for (int w2 = 0; w2 < kRowWaves; ++w2)
            t_lo = w2 == 0 ? first_tile[0] : min(t_lo, first_tile[w2]);
    }

    // per wave: 256-bin histogram, cap keys, cap 16-bit entries
    TopKRow<uint16_t> tk;
    if (MODE & kModeSelect) {
        unsigned char *base = smem + 2 * G::kTileBytes + (size_t)wv * rows_topk_wave_bytes(a.cap);
        uint32_t *hist = reinterpret_cast<uint32_t *>(base);
        uint32_t *key = hist + 256;
        topk_init(tk, key, reinterpret_cast<uint16_t *>(key + a.cap + kWave), hist, a.cap, a.top_k);
    }

    // Key tiles arrive by DMA (no registers, no address arithmetic per tile):
    // the buffer resource covers the tile's entries that exist, so slots of
    // entries at or past W read zeros (those entries are always masked).
    const uint16_t *kb = a.k + b * a.k_sb;
    const int entry_bytes = (int)a.k_sw * 2;
    const int64_t tile_stride = (int64_t)kTileEntries * a.k_sw;
    const int W = a.W;
    uint32_t dma_off[G::kDmaPerWave];
#pragma unroll
    for (int x = 0; x < G::kDmaPerWave; ++x) {
        const int slot = (wv + x * kRowWaves) * kWave + l;
        dma_off[x] = (uint32_t)((slot / G::kRowChunks) * entry_bytes + (slot % G::kRowChunks) * 16);
    }
    // ops wv, wv+4, ...: all waves have the first kDmaOps / 4, the first
    // kDmaOps % 4 waves one more
    constexpr int kFullOps = G::kDmaOps / kRowWaves;
    const bool extra_op = wv < G::kDmaOps % kRowWaves;
    auto fetch = [&](int t) {
        const int e0 = t * kTileEntries;
        const int n = min(W - e0, kTileEntries);
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(kb + t * tile_stride, entries_span<D>(n, entry_bytes));
        unsigned char *dst = smem + (size_t)(t & 1) * G::kTileBytes + wv * kWave * 16;
#pragma unroll
        for (int x = 0; x < kFullOps; ++x)
            dma16(r, dst + x * kRowWaves * kWave * 16, dma_off[x]);
        if (kFullOps < G::kDmaPerWave && extra_op)
            dma16(r, dst + kFullOps * kRowWaves * kWave * 16, dma_off[G::kDmaPerWave - 1]);
    };
    KLAcc klacc = kl_empty();
    const float *tgt_row = (MODE & kModeKL) && active ? a.target + row_id * a.W : nullptr;
    // this lane's target weight of tile tt (any value for entries past W)
    auto tgt_load = [&](int tt) -> float {
        if (!(MODE & kModeKL) || !active)
            return 0.0f;
        return tgt_row[min(tt * kTileEntries + l, a.W - 1)];
    };
    auto emit = [&](int tt, float s, bool valid, float tgt) {
        const int j = tt * kTileEntries + l;
        const float outv = valid ? s : -INFINITY;
        if (MODE & kModeScores) {
            if (j < a.W)
                a.scores[row_id * a.W + j] = outv;
        }
        if (MODE & kModeSelect)
            topk_push_unchecked(tk, score_key(outv), (uint32_t)j, valid);
        if (MODE & kModeKL) {
            if (valid)
                kl_add(klacc, s, tgt);
        }
    };
    auto tile_valid = [&](int tt) {
        const int j = tt * kTileEntries + l;
        bool v = j < thr;
        if (kseg)
            v = v && kseg[min(j, a.W - 1)] == qseg;
        return v;
    };

    // The first key tile's DMA goes out before the row operands' loads so the
    // two latencies overlap.  Each iteration then waits for its own DMA,
    // meets the other waves at the barrier (tile t complete, tile t-1's buffer
    // free) and starts the DMA of tile t+1 into that buffer.
    if (ntiles > t_lo)
        fetch(t_lo);
    RowOperand<HB, KS> row;
    if (active)
        load_row<HB, KS>(row, a.q + b * a.q_sb + (int64_t)i * a.q_ss, a.q_sh, a.w + b * a.w_sb + (int64_t)i * a.w_ss,
                         a.H);
    for (int t = t_lo; t < ntiles; ++t) {
        wait_vm();
        __syncthreads();
        if (t + 1 < ntiles)
            fetch(t + 1);
        if (active) {
            const uint16_t *tile = ktile + (t & 1) * G::kTileElems;
            const bool valid = tile_valid(t);
            const float tgt_cur = tgt_load(t);
            const float s = tile_scores<HB, KS>(row, true, true, a.scale, [&](bf16x8(&bf)[KS], int sub) {
                load_entries_lds<KS>(bf, tile, sub * 32, G::kPitch);
            });
            if (MODE & kModeSelect)
                topk_reserve(tk);
            emit(t, s, valid, tgt_cur);
        }
    }
    if (active && (MODE & kModeScores)) {
        // entries before the first computed tile are masked
        for (int j = l; j < min(t_lo * kTileEntries, a.W); j += kWave)
            a.scores[row_id * a.W + j] = -INFINITY;
    }

    if (!active)
        return;
    if (MODE & kModeScores) {
        for (int j = max(ntiles, t_lo) * kTileEntries + l; j < a.W; j += kWave)
            a.scores[row_id * a.W + j] = -INFINITY;
    }
    if (MODE & kModeSelect) {
        // buffers of up to 1536 pairs (k <= 512) finish from registers
        if (a.cap <= 24 * kWave)
            topk_finish_regs<24>(tk, a.idx + row_id * a.top_k);
        else
            topk_finish(tk, a.idx + row_id * a.top_k);
    }
    if (MODE & kModeKL) {
        const KLAcc tot = kl_wave_reduce(klacc);
        if (l == 0)
            a.kl[row_id] = kl_value(tot);
    }
}

// ---------------------------------------------------------------------------
// Row-tile plan for up to 64 heads: three workgroups per compute unit (three
// waves per SIMD), so that while one wave is in its epilogue, its top-k
// bookkeeping or the final selection, two others keep the matrix core busy.
// That budget (at most 168 VGPRs, 53 KB of LDS per workgroup) shapes the
// loop: key tiles of 32 entries (double-buffered, one barrier per tile), the
// B fragments of a tile read from LDS three k-steps ahead of their MFMAs
// instead of all at once, one accumulator set per wave (the ReLU·w epilogue
// of a tile follows its MFMAs; the other waves fill the matrix core
// meanwhile), and a candidate buffer of k + 704 pairs.  Pairs of tiles make
// the 64-entry units whose scores are pushed, written or folded (one score
// per lane); segment skipping works on those units.  Everything else --
// operands, masks, the order of operations, hence the bits -- is that of
// rows_kernel.
// ---------------------------------------------------------------------------
constexpr int kTile3 = 32;

template <int D>
struct Tile3Geom {
    static constexpr int kKs = D / 16;
    static constexpr int kPitch = D + 8;                            // LDS row pitch (elements)
    static constexpr int kRowChunks = kPitch / 8;                   // 16-byte slots per row
    static constexpr int kDmaOps = (kTile3 * kRowChunks + kWave - 1) / kWave;
    static constexpr int kDmaPerWave = (kDmaOps + kRowWaves - 1) / kRowWaves;
    static constexpr size_t kBufBytes = (size_t)kDmaOps * kWave * 16; // whole DMA instructions
};

template <int D, int HB, int MODE>
__global__ __launch_bounds__(kRowWaves * kWave) __attribute__((amdgpu_waves_per_eu(3)))
void rows3_kernel(const KernelArgs a)
{
    using G = Tile3Geom<D>;
    constexpr int KS = G::kKs;
    static_assert(HB <= 2, "three waves per SIMD hold at most two head blocks");
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x;
    const int wv = uniform(tid / kWave);
    const int l = lane();

    const int W = own_sgpr(a.W), top_k = own_sgpr(a.top_k), cap = own_sgpr(a.cap);
    const int rb = a.n_row_blocks - 1 - (int)(blockIdx.x / a.B);
    const int b = (int)(blockIdx.x % a.B);
    const int row0 = rb * kRowsPerBlock;
    const int i = row0 + wv;
    const bool active = i < a.S;

    const int64_t off = a.q_offset ? (int64_t)a.q_offset[b] : 0;
    const int last = min(row0 + kRowsPerBlock, a.S) - 1;
    const int thr_last = visible_entries(off + last, a.m, W);
    const int nunits = (thr_last + kTileEntries - 1) / kTileEntries; // 64-entry units
    const int ntiles = (thr_last + kTile3 - 1) / kTile3;             // 32-entry tiles
    const int thr = active ? visible_entries(off + i, a.m, W) : 0;
    constexpr bool kSegs = (MODE & kModeSegs) != 0;
    const int qseg = (kSegs && active) ? a.q_seg[(int64_t)b * a.S + i] : 0;
    const int32_t *kseg = kSegs ? a.k_seg + (int64_t)b * W : nullptr;
    const int64_t row_id = (int64_t)b * a.S + i;

    // With segments, units before the first one that holds an entry of any
    // row's segment are masked for the whole workgroup and are skipped.
    int u_lo = 0;
    if (kSegs) {
        __shared__ int first_unit[kRowWaves];
        const int fu = active ? first_segment_unit(kseg, thr, qseg, nunits, W) : nunits;
        if (l == 0)
            first_unit[wv] = fu;
        __syncthreads();
#pragma unroll
        for (int w2 = 0; w2 < kRowWaves; ++w2)
            u_lo = w2 == 0 ? first_unit[0] : min(u_lo, first_unit[w2]);
    }

    TopKRow<uint16_t> tk;
    if (MODE & kModeSelect) {
        unsigned char *base = smem + 2 * G::kBufBytes + (size_t)wv * rows_topk_wave_bytes(cap);
        uint32_t *hist = reinterpret_cast<uint32_t *>(base);
        uint32_t *key = hist + 256;
        topk_init(tk, key, reinterpret_cast<uint16_t *>(key + cap + kWave), hist, cap, top_k);
    }

    // Key tiles by DMA, as in rows_kernel: DMA instruction o of a tile writes
    // the 64 16-byte slots 64o .. 64o+63 of the padded image; slots past the
    // tile's entries (and past W) read zeros and are never consumed.
    const uint16_t *kb = a.k + b * a.k_sb;
    const int entry_bytes = (int)a.k_sw * 2;
    const int64_t tile_stride = (int64_t)kTile3 * a.k_sw;
    uint32_t dma_off[G::kDmaPerWave];
#pragma unroll
    for (int x = 0; x < G::kDmaPerWave; ++x) {
        const int slot = (wv + x * kRowWaves) * kWave + l;
        dma_off[x] = (uint32_t)((slot / G::kRowChunks) * entry_bytes + (slot % G::kRowChunks) * 16);
    }
    auto fetch = [&](int t) {
        const int n = min(W - t * kTile3, kTile3);
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(kb + t * tile_stride, entries_span<D>(n, entry_bytes));
        unsigned char *dst = smem + (size_t)(t & 1) * G::kBufBytes + wv * kWave * 16;
#pragma unroll
        for (int x = 0; x < G::kDmaPerWave; ++x)
            if (wv + x * kRowWaves < G::kDmaOps)
                dma16(r, dst + x * kRowWaves * kWave * 16, dma_off[x]);
    };

    KLAcc klacc = kl_empty();
    const float *tgt_row = (MODE & kModeKL) && active ? a.target + row_id * W : nullptr;
    auto tgt_load = [&](int u) -> float {
        if (!(MODE & kModeKL) || !active)
            return 0.0f;
        return tgt_row[min(u * kTileEntries + l, W - 1)];
    };
    // segment id of this lane's entry of unit u (loaded at the unit's first
    // tile, compared at its last, so the load's latency is hidden)
    auto seg_load = [&](int u) -> int { return kSegs ? kseg[min(u * kTileEntries + l, W - 1)] : 0; };
    auto unit_valid = [&](int u, int seg) {
        const int j = u * kTileEntries + l;
        bool v = j < thr;
        if (kSegs)
            v = v && seg == qseg;
        return v;
    };
    auto emit = [&](int u, float s, bool valid, float tgt) {
        const int j = u * kTileEntries + l;
        const float outv = valid ? s : -INFINITY;
        if (MODE & kModeScores) {
            if (j < W)
                a.scores[row_id * W + j] = outv;
        }
        // a masked entry carries the key of -inf, which never exceeds tau
        if (MODE & kModeSelect)
            topk_push_unchecked(tk, score_key(outv), (uint32_t)j, true);
        if (MODE & kModeKL) {
            if (valid)
                kl_add(klacc, s, tgt);
        }
    };

    const int t_lo = 2 * u_lo;
    if (ntiles > t_lo)
        fetch(t_lo);
    RowOperand<HB, KS> row;
    if (active)
        load_row<HB, KS>(row, a.q + b * a.q_sb + (int64_t)i * a.q_ss, a.q_sh, a.w + b * a.w_sb + (int64_t)i * a.w_ss,
                         a.H);
    // this lane's B fragment of k-step s: entry (l % 32), values 16s + 8(l / 32)
    const int boff = (l & 31) * G::kPitch + 8 * (l >> 5);
    float p_even = 0.0f, tgt_unit = 0.0f;
    int seg_unit = 0;
    for (int t = t_lo; t < ntiles; ++t) {
        wait_vm();
        __syncthreads();
        if (t + 1 < ntiles)
            fetch(t + 1);
        if (active) {
            const uint16_t *tile = reinterpret_cast<const uint16_t *>(smem + (size_t)(t & 1) * G::kBufBytes);
            if ((t & 1) == 0) {
                tgt_unit = tgt_load(t >> 1);
                seg_unit = seg_load(t >> 1);
            }
            f32x16 c[HB];
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
                c[hb] = f32x16{};
            constexpr int kAhead = KS < 3 ? KS : 3;
            bf16x8 bq[kAhead];
#pragma unroll
            for (int s2 = 0; s2 < kAhead; ++s2)
                bq[s2] = load_frag(tile + boff + 16 * s2);
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
#pragma unroll
                for (int hb = 0; hb < HB; ++hb)
                    c[hb] = mfma32(row.a[hb][s2], bq[s2 % kAhead], c[hb]);
                if (s2 + kAhead < KS)
                    bq[s2 % kAhead] = load_frag(tile + boff + 16 * (s2 + kAhead));
            }
            const float p = logits_partial<HB, KS>(row, c);
            if ((t & 1) == 0 && t + 1 < ntiles) {
                p_even = p;
            } else {
                // a 64-entry unit is complete: entries of the odd tile (or
                // none past an even last tile) sit in the upper lane half
                const int u = t >> 1;
                const bool odd = (t & 1) != 0;
                const float sc = scaled_score(combine_halves(odd ? p_even : p, odd ? p : 0.0f), a.scale);
                const bool valid = unit_valid(u, seg_unit);
                if (MODE & kModeSelect)
                    topk_reserve(tk);
                emit(u, sc, valid, tgt_unit);
            }
        }
    }
    if (!active)
        return;
    if (MODE & kModeScores) {
        // entries before the first computed unit and past the last are masked
        for (int j = l; j < min(u_lo * kTileEntries, W); j += kWave)
            a.scores[row_id * W + j] = -INFINITY;
        for (int j = max(nunits, u_lo) * kTileEntries + l; j < W; j += kWave)
            a.scores[row_id * W + j] = -INFINITY;
    }
    if (MODE & kModeSelect) {
        if (cap <= 24 * kWave)
            topk_finish_regs<24>(tk, a.idx + row_id * top_k);
        else
            topk_finish(tk, a.idx + row_id * top_k);
    }
    if (MODE & kModeKL) {
        const KLAcc tot = kl_wave_reduce(klacc);
        if (l == 0)
            a.kl[row_id] = kl_value(tot);
    }
}

// ---------------------------------------------------------------------------
// Split-row plan (long rows, few of them: decode).  Workgroup (row, chunk)
// scores kSplitChunk consecutive entries of one row; each wave takes
// kSplitTiles tiles of 64 entries.  Every key byte is used by one row only,
// so nothing is shared through LDS: each wave stages its own 32-entry
// subtiles there by DMA (coalesced 16-byte slots, double-buffered, the next
// subtile in flight while the current one is computed) and reads its MFMA
// fragments back.  Only the visible prefix of the row is read (the DMA's
// buffer resource ends there, so entries past it read zeros and are masked).
// Scores go to a.scores with row stride W; with full_rows the rest of the row
// is filled with -inf.
// ---------------------------------------------------------------------------
template <int D>
struct SplitGeom {
    static constexpr int kPitch = D + 8;                          // elements per LDS row
    static constexpr int kRowChunks = kPitch / 8;                 // 16-byte slots per row
    static constexpr int kSlots = 32 * kRowChunks;                // slots of one subtile
    static constexpr int kDmaOps = (kSlots + kWave - 1) / kWave;  // DMA instructions per subtile
    static constexpr int kBufBytes = kDmaOps * kWave * 16;        // subtile buffer (whole DMA ops)
    static constexpr int kWaveBytes = 2 * kBufBytes;
};

template <int D, int HB>
__global__ __launch_bounds__(kSplitWaves * kWave) void split_kernel(const KernelArgs a)
{
    using G = SplitGeom<D>;
    constexpr int KS = D / 16;
    constexpr int kWaveEntries = kSplitTiles * kTileEntries;
    constexpr int kSubtiles = 2 * kSplitTiles;
    extern __shared__ __align__(16) unsigned char smem[];
    const int wv = uniform(threadIdx.x / kWave);
    const int l = lane();
    // chunk-major order: every row's first chunks are dispatched before any
    // row's last ones (which are empty for short rows), and the row of a
    // given position rotates with the chunk so consecutive workgroups (which
    // land on different XCDs) do not keep the same rows
    const int64_t chunk = (int64_t)blockIdx.x / a.rows;
    const int64_t row_id = ((int64_t)blockIdx.x % a.rows + chunk) % a.rows;
    const int b = (int)(row_id / a.S), i = (int)(row_id % a.S);
    const int64_t off = a.q_offset ? (int64_t)a.q_offset[b] : 0;
    const int thr = visible_entries(off + i, a.m, a.W);
    const int base = (int)chunk * kSplitChunk + wv * kWaveEntries;
    float *out = a.scores + row_id * a.W;

    if (base >= thr) {
        if (a.full_rows)
            for (int j = base + l; j < min(base + kWaveEntries, a.W); j += kWave)
                out[j] = -INFINITY;
        return;
    }
    const int qseg = a.q_seg ? a.q_seg[row_id] : 0;
    const int32_t *kseg = a.k_seg ? a.k_seg + (int64_t)b * a.W : nullptr;

    // subtile DMA: slot x*64 + l holds chunk slot % kRowChunks of entry
    // slot / kRowChunks (slots past the 32 entries read zeros)
    const int entry_bytes = (int)a.k_sw * 2;
    const uint16_t *kb = a.k + b * a.k_sb;
    unsigned char *wbuf = smem + (size_t)wv * G::kWaveBytes;
    auto dma_subtile = [&](int sub) {
        const int e0 = base + sub * 32;
        const int n = max(0, min(32, thr - e0));
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(kb + (int64_t)e0 * a.k_sw, entries_span<D>(n, entry_bytes));
        unsigned char *dst = wbuf + (sub & 1) * G::kBufBytes;
#pragma unroll
        for (int x = 0; x < G::kDmaOps; ++x) {
            const int slot = x * kWave + l;
            dma16(r, dst + x * kWave * 16,
                  (uint32_t)((slot / G::kRowChunks) * entry_bytes + (slot % G::kRowChunks) * 16));
        }
    };
    const int nsub = min(kSubtiles, (thr - base + 31) / 32);

    // Two subtiles stay in flight: a buffer is refilled as soon as its
    // fragments are in registers.  Issue order per iteration s: the previous
    // tile's score store (if any), then DMA(s+2), so when iteration s waits
    // for DMA(s) the younger vector-memory ops are exactly DMA(s+1) and the
    // store issued in iteration s-1, and the wait names that count.
    auto score_store = [&](int tile_j0, float pa, float pb) {
        const int j = tile_j0 + l;
        bool valid = j < thr;
        if (kseg)
            valid = valid && kseg[min(j, a.W - 1)] == qseg;
        const float sc = scaled_score(combine_halves(pa, pb), a.scale);
        if (j < a.W && (a.full_rows || j < thr))
            out[j] = valid ? sc : -INFINITY;
    };
    dma_subtile(0);
    RowOperand<HB, KS> row;
    load_row<HB, KS>(row, a.q + b * a.q_sb + (int64_t)i * a.q_ss, a.q_sh, a.w + b * a.w_sb + (int64_t)i * a.w_ss, a.H);
    if (nsub > 1)
        dma_subtile(1);

    float p0 = 0.0f, pend_a = 0.0f, pend_b = 0.0f;
    bool pend = false;
#pragma unroll 1
    for (int sub = 0; sub < nsub; ++sub) {
        // wait for DMA(sub): younger ops are DMA(sub+1) (if issued) and the
        // store of iteration sub-1 (if any)
        // (with segments the store also loads segment ids: wait for all)
        const bool younger_dma = sub + 1 < nsub && !kseg;
        const bool younger_store = sub >= 3 && (sub & 1) == 1;
        if (younger_dma && younger_store)
            vm_wait_le<G::kDmaOps + 1>();
        else if (younger_dma)
            vm_wait_le<G::kDmaOps>();
        else
            wait_vm();
        bf16x8 bf[KS];
        load_entries_lds<KS>(bf, reinterpret_cast<const uint16_t *>(wbuf + (sub & 1) * G::kBufBytes), 0, G::kPitch);
        lds_wait();
        __asm__ volatile("" ::: "memory");
        if (pend) {
            score_store(base + (sub - 2) * 32, pend_a, pend_b);
            pend = false;
        }
        __asm__ volatile("" ::: "memory");
        if (sub + 2 < nsub)
            dma_subtile(sub + 2);
        __asm__ volatile("" ::: "memory");
        const float p = subtile_partial<HB, KS>(row, bf);
        if (sub & 1) {
            pend_a = p0;
            pend_b = p;
            pend = true;
        } else {
            p0 = p;
        }
    }
    if (pend)
        score_store(base + (nsub - 2) * 32, pend_a, pend_b);
    if (nsub & 1) // the last 64-entry tile has only its first half computed
        score_store(base + (nsub - 1) * 32, p0, 0.0f);
    if (a.full_rows)
        for (int j = base + ((nsub + 1) / 2) * kTileEntries + l; j < min(base + kWaveEntries, a.W); j += kWave)
            out[j] = -INFINITY;
}

// ---------------------------------------------------------------------------
// Balanced split plan (few rows, scores to the workspace: decode).  The
// visible prefixes of all rows, cut into 64-entry tiles and laid end to end,
// are divided into equal contiguous ranges, one per wave of a grid sized to
// the chip, so every wave streams the same number of key bytes whatever the
// row lengths are.  A wave walks its range tile by tile, crossing into the
// next row where one ends (it then loads that row's query fragments and
// weights); its key subtiles are staged by DMA exactly as in split_kernel,
// two in flight.  Only visible entries are written.  Ranges are assigned so
// that consecutive ranges (which mostly share a row) go to workgroups on the
// same XCD.
// ---------------------------------------------------------------------------
constexpr int kStreamMaxRows = kStreamRows;
// rows per thread in the workgroup's prefix over rows, and the slots it fills
constexpr int kStreamPer = (kStreamMaxRows + kStreamWaves * kWave - 1) / (kStreamWaves * kWave);
constexpr int kStreamSlots = kStreamPer * kStreamWaves * kWave;
static_assert(kStreamSlots >= kStreamMaxRows, "every row has a slot");

// Two waves per SIMD: without the bound the compiler takes all 256 VGPRs and
// some accumulation registers besides, which leaves one wave per SIMD.
template <int D, int HB>
__global__ __launch_bounds__(kStreamWaves * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void stream_kernel(const KernelArgs a)
{
    using G = SplitGeom<D>;
    constexpr int KS = D / 16;
    constexpr int kPer = kStreamPer;
    extern __shared__ __align__(16) unsigned char smem[];
    int *pre = reinterpret_cast<int *>(smem + kStreamWaves * G::kWaveBytes); // [kStreamSlots + 1]
    int *thr_of = pre + kStreamSlots + 1;                                    // [kStreamSlots]
    __shared__ int wsum[kStreamWaves];
    const int tid = threadIdx.x;
    const int wv = uniform(tid / kWave);
    const int l = lane();
    const int rows = (int)a.rows;

    // tiles per row and their exclusive prefix (row-major order); slots past
    // the last row hold the total
    int cnt[kPer], tot = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int row = tid * kPer + r;
        int t = 0;
        if (row < rows) {
            const int b = row / a.S, i = row % a.S;
            t = visible_entries((a.q_offset ? (int64_t)a.q_offset[b] : 0) + i, a.m, a.W);
            thr_of[row] = t;
        }
        cnt[r] = (t + kTileEntries - 1) / kTileEntries;
        tot += cnt[r];
    }
    const int incl = wave_inclusive_sum(tot);
    if (l == kWave - 1)
        wsum[wv] = incl;
    __syncthreads();
    int before = incl - tot, total = 0;
#pragma unroll
    for (int w2 = 0; w2 < kStreamWaves; ++w2) {
        before += w2 < wv ? wsum[w2] : 0;
        total += wsum[w2];
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        pre[tid * kPer + r] = before;
        before += cnt[r];
    }
    if (tid == 0)
        pre[kStreamSlots] = total;
    __syncthreads();
    // this wave's range of tiles [t0, t1)
    const int nblk = (int)gridDim.x;
    const int blk = (nblk % 8 == 0) ? (int)(blockIdx.x % 8) * (nblk / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int64_t gw = (int64_t)blk * kStreamWaves + wv, nw = (int64_t)nblk * kStreamWaves;
    const int t0 = (int)((int64_t)total * gw / nw), t1 = (int)((int64_t)total * (gw + 1) / nw);
    // Subtiles each wave has left, for the priority balance below (waves w
    // and w ^ 4 share a SIMD).
    static_assert(kStreamWaves == 8, "two waves per SIMD");
    __shared__ int left[kStreamWaves];
    if (l == 0)
        left[wv] = 2 * max(t1 - t0, 0);
    if (t0 >= t1)
        return;
    // row holding tile t0: the last row r with pre[r] <= t0 (rows before it
    // that have no tiles share its prefix and are passed over)
    int lo = 0, hi = rows; // invariant: pre[lo] <= t0 < pre[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= t0)
            lo = mid;
        else
            hi = mid;
    }

    // Cursor over tiles: row, first tile of the row, end of the row's tiles.
    struct Cursor {
        int row, rs, re;
    };
    auto next_row = [&](Cursor &c) {
        do {
            ++c.row;
        } while (c.row < rows && pre[c.row + 1] == pre[c.row]);
        c.rs = pre[c.row];
        c.re = c.row < rows ? pre[c.row + 1] : c.rs;
    };
    Cursor dc{lo, pre[lo], pre[lo + 1]}; // DMA cursor (runs up to two subtiles ahead)
    const int entry_bytes = (int)a.k_sw * 2;
    unsigned char *wbuf = smem + (size_t)wv * G::kWaveBytes;
    // DMA of subtile `sub` of this wave (tile t0 + sub/2); advances dc past
    // the tile after its second half
    auto dma_subtile = [&](int sub) {
        const int t = t0 + (sub >> 1);
        if (t >= dc.re)
            next_row(dc);
        const int b = dc.row / a.S;
        const int e0 = (t - dc.rs) * kTileEntries + (sub & 1) * 32;
        const int n = max(0, min(32, thr_of[dc.row] - e0));
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(a.k + b * a.k_sb + (int64_t)e0 * a.k_sw, entries_span<D>(n, entry_bytes));
        unsigned char *dst = wbuf + (sub & 1) * G::kBufBytes;
#pragma unroll
        for (int x = 0; x < G::kDmaOps; ++x) {
            const int slot = x * kWave + l;
            dma16(r, dst + x * kWave * 16,
                  (uint32_t)((slot / G::kRowChunks) * entry_bytes + (slot % G::kRowChunks) * 16));
        }
    };
    const int nsub = 2 * (t1 - t0);
    dma_subtile(0);
    dma_subtile(1);

    Cursor cc{lo - 1, 0, t0}; // compute cursor: entered its first row below
    RowOperand<HB, KS> row;
    int thr = 0, qseg = 0;
    const int32_t *kseg = nullptr;
    float *out = nullptr;
    float p0 = 0.0f;
    // pending store: the previous tile's partials and where they go
    float pend_a = 0.0f, pend_b = 0.0f;
    bool pend = false;
    float *pend_out = nullptr;
    int pend_j0 = 0, pend_thr = 0, pend_qseg = 0;
    const int32_t *pend_kseg = nullptr;
    auto score_store = [&](float *o, int j0, int th, const int32_t *ks, int qs, float pa, float pb) {
        const int j = j0 + l;
        bool valid = j < th;
        if (ks)
            valid = valid && ks[min(j, a.W - 1)] == qs;
        const float sc = scaled_score(combine_halves(pa, pb), a.scale);
        if (j < th)
            o[j] = valid ? sc : -INFINITY;
    };
    const bool segs = a.k_seg != nullptr;
#pragma unroll 1
    for (int sub = 0; sub < nsub; ++sub) {
        const int t = t0 + (sub >> 1);
        bool switched = false;
        if ((sub & 1) == 0 && t >= cc.re) {
            next_row(cc);
            switched = true;
        }
        if (switched) {
            // new row: its operands, then everything outstanding
            const int b = cc.row / a.S, i = cc.row % a.S;
            load_row<HB, KS>(row, a.q + b * a.q_sb + (int64_t)i * a.q_ss, a.q_sh,
                             a.w + b * a.w_sb + (int64_t)i * a.w_ss, a.H);
            thr = thr_of[cc.row];
            kseg = segs ? a.k_seg + (int64_t)b * a.W : nullptr;
            qseg = segs ? a.q_seg[cc.row] : 0;
            out = a.scores + (int64_t)cc.row * a.W;
            wait_vm();
        } else {
            // younger vector-memory ops than DMA(sub): DMA(sub+1) if issued,
            // and the store issued in the previous iteration if any (stores
            // go out in even iterations from the fourth subtile on)
            const bool younger_dma = sub + 1 < nsub && !segs;
            const bool younger_store = sub >= 3 && (sub & 1) == 1;
            if (younger_dma && younger_store)
                vm_wait_le<G::kDmaOps + 1>();
            else if (younger_dma)
                vm_wait_le<G::kDmaOps>();
            else
                wait_vm();
        }
        bf16x8 bf[KS];
        load_entries_lds<KS>(bf, reinterpret_cast<const uint16_t *>(wbuf + (sub & 1) * G::kBufBytes), 0, G::kPitch);
        // The two waves of a SIMD (w and w ^ 4) have equal shares, but the
        // older one wins the issue arbitration and would finish well ahead:
        // the wave with more subtiles left takes the higher priority.
        if (l == 0)
            left[wv] = nsub - sub;
        const int partner_left = left[wv ^ 4];
        lds_wait();
        if (nsub - sub > uniform(partner_left))
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
        __asm__ volatile("" ::: "memory");
        if (pend) {
            score_store(pend_out, pend_j0, pend_thr, pend_kseg, pend_qseg, pend_a, pend_b);
            pend = false;
        }
        __asm__ volatile("" ::: "memory");
        if (sub + 2 < nsub)
            dma_subtile(sub + 2);
        __asm__ volatile("" ::: "memory");
        const float p = subtile_partial<HB, KS>(row, bf);
        if (sub & 1) {
            pend_a = p0;
            pend_b = p;
            pend = true;
            pend_out = out;
            pend_j0 = (t - cc.rs) * kTileEntries;
            pend_thr = thr;
            pend_kseg = kseg;
            pend_qseg = qseg;
        } else {
            p0 = p;
        }
    }
    if (pend)
        score_store(pend_out, pend_j0, pend_thr, pend_kseg, pend_qseg, pend_a, pend_b);
}

// ---------------------------------------------------------------------------
// Row top-k over a dense fp32 score matrix, one wave per row (short rows).
// With limit_rows the row ends at its visible prefix (q_offset, m).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int row_length(const KernelArgs &a, int64_t row)
{
    if (!a.limit_rows)
        return a.W;
    const int b = (int)(row / a.S), i = (int)(row % a.S);
    const int64_t off = a.q_offset ? (int64_t)a.q_offset[b] : 0;
    return visible_entries(off + i, a.m, a.W);
}

// Stream src[j0 .. j1) (j1 - j0 a multiple of 64 or the row end n) into the
// wave's buffer, sixteen 64-entry chunks per batch of loads.
__device__ __forceinline__ void stream_row(TopKRow<uint32_t> &tk, const float *src, int j0, int j1, int n)
{
    const int l = lane();
    constexpr int kBatch = 16;
#pragma unroll 1
    for (int base = j0; base < j1; base += kBatch * kWave) {
        float v[kBatch];
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int j = base + c * kWave + l;
            v[c] = src[min(j, n - 1)];
        }
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int j = base + c * kWave + l;
            const bool in = j < j1;
            const uint32_t kv = score_key(v[c]);
            topk_push(tk, kv, (uint32_t)j, in && key_selectable(kv));
        }
    }
}

__global__ __launch_bounds__(kTopkWaves * kWave) void topk_kernel(const KernelArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int wv = uniform(threadIdx.x / kWave);
    const int64_t row = (int64_t)blockIdx.x * kTopkWaves + wv;
    if (row >= a.rows)
        return;
    if (a.redo && a.idx[row * a.top_k] != kTopkRedo)
        return; // the workgroup-per-row kernel selected this row
    const int n = row_length(a, row);
    unsigned char *base = smem + (size_t)wv * (1024 + (size_t)a.cap * 8);
    uint32_t *hist = reinterpret_cast<uint32_t *>(base);
    uint32_t *key = hist + 256;
    TopKRow<uint32_t> tk;
    topk_init(tk, key, key + a.cap, hist, a.cap, a.top_k);
    if (n > 0)
        stream_row(tk, a.scores + row * a.W, 0, n, n);
    topk_finish(tk, a.idx + row * a.top_k);
}

// ---------------------------------------------------------------------------
// Row top-k for long rows: one workgroup per row.  Rows whose keys fit in
// LDS take the fast path below (topk_block_fast); the others, and the rows
// it declines, take the streaming path: a first pass builds a histogram of
// the row's keys by their top kCoarseBits bits and finds the bucket holding
// the k-th largest key: every key below that bucket is beaten by at least k
// others, so the waves start with tau just below it and their buffers only
// ever see the few keys at or above it.  Wave w then streams the w-th
// contiguous segment into its own buffer, and the waves select jointly.
// ---------------------------------------------------------------------------
constexpr int kCoarseBits = 12;
constexpr int kCoarseBins = 1 << kCoarseBits;

template <int NW>
__device__ __forceinline__ void coarse_clear(uint32_t *hist)
{
    for (int b = threadIdx.x; b < kCoarseBins; b += NW * kWave)
        hist[b] = 0u;
}

__device__ __forceinline__ void coarse_add(uint32_t *hist, uint32_t kv)
{
    if (key_selectable(kv))
        atomicAdd(&hist[kv >> (32 - kCoarseBits)], 1u);
}

// The bin holding the k-th largest count of a complete histogram, counting
// from the top bin down (-1 when the bins hold fewer than k).  All threads
// of the workgroup call it; `part` is NW+1 words.
template <int NW>
__device__ __forceinline__ int coarse_find_bin(const uint32_t *hist, int k, int *part)
{
    constexpr int kThreads = NW * kWave;
    // thread t owns bins kCoarseBins-1-t*P .. (descending), P bins each
    constexpr int P = kCoarseBins / kThreads;
    const int wv = threadIdx.x / kWave;
    int h[P], tot = 0;
#pragma unroll
    for (int r = 0; r < P; ++r) {
        h[r] = (int)hist[kCoarseBins - 1 - threadIdx.x * P - r];
        tot += h[r];
    }
    const int incl = wave_inclusive_sum(tot);
    if (lane() == kWave - 1)
        part[wv] = incl;
    __syncthreads();
    int before = incl - tot;
    for (int w = 0; w < wv; ++w)
        before += part[w];
    if (threadIdx.x == 0)
        part[NW] = -1;
    __syncthreads();
    int cum = before;
#pragma unroll
    for (int r = 0; r < P; ++r) {
        if (cum < k && k <= cum + h[r])
            part[NW] = kCoarseBins - 1 - (int)threadIdx.x * P - r; // unique: cumulative counts are monotone
        cum += h[r];
    }
    __syncthreads();
    const int bin = part[NW];
    __syncthreads();
    return bin;
}

// Key below which no key of the row can make its top k: one less than the
// lower bound of the bucket that holds the k-th largest selectable key
// (kKeyNegInf when the row has fewer than k of them).
__device__ __forceinline__ uint32_t coarse_tau(int bin)
{
    return bin <= 0 ? kKeyNegInf : max(((uint32_t)bin << (32 - kCoarseBits)) - 1u, kKeyNegInf);
}

// The same from the row in global memory (one read pass).
template <int NW>
__device__ __forceinline__ uint32_t coarse_threshold(const float *src, int n, int k, uint32_t *hist, int *part)
{
    constexpr int kThreads = NW * kWave;
    coarse_clear<NW>(hist);
    __syncthreads();
    const int n4 = n / 4;
    const float4 *src4 = reinterpret_cast<const float4 *>(src);
    const bool vec = (reinterpret_cast<uintptr_t>(src) & 15u) == 0;
    const int nv = vec ? n4 : 0;
    // batches of 8 float4 per thread, all loads of a batch in flight at once
    constexpr int kB = 8;
#pragma unroll 1
    for (int i0 = 0; i0 < nv; i0 += kB * kThreads) {
        float4 v[kB];
#pragma unroll
        for (int x = 0; x < kB; ++x) {
            const int i = i0 + x * kThreads + (int)threadIdx.x;
            v[x] = i < nv ? src4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
#pragma unroll
        for (int x = 0; x < kB; ++x) {
            coarse_add(hist, score_key(v[x].x));
            coarse_add(hist, score_key(v[x].y));
            coarse_add(hist, score_key(v[x].z));
            coarse_add(hist, score_key(v[x].w));
        }
    }
    for (int j = nv * 4 + threadIdx.x; j < n; j += kThreads)
        coarse_add(hist, score_key(src[j]));
    __syncthreads();
    return coarse_tau(coarse_find_bin<NW>(hist, k, part));
}

// Fast path of the long-row top-k for rows of at most kTopkBlockFastMaxW
// entries: the row is read once from global memory into LDS as keys, with the
// coarse histogram built on the way; its bucket of the k-th largest key (split
// once more by the next key bits when it holds too many) bounds the
// candidates, usually a few hundred, which are compacted into LDS; the waves
// sort them as 64-bit composites (key, ~entry), so that equal keys come out
// in entry order, and the first k sorted positions are the selection.
// Returns false, having written nothing, when there are more than
// kBlockCandMax candidates.
constexpr int kBlockCandMax = 2048;

__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v, int lx)
{
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    switch (lx) {
    case 1: lo = lane_xor_u32<1>(lo); hi = lane_xor_u32<1>(hi); break;
    case 2: lo = lane_xor_u32<2>(lo); hi = lane_xor_u32<2>(hi); break;
    case 4: lo = lane_xor_u32<4>(lo); hi = lane_xor_u32<4>(hi); break;
    case 8: lo = lane_xor_u32<8>(lo); hi = lane_xor_u32<8>(hi); break;
    case 16: lo = lane_xor_u32<16>(lo); hi = lane_xor_u32<16>(hi); break;
    default: lo = lane_xor_u32<32>(lo); hi = lane_xor_u32<32>(hi); break;
    }
    return ((uint64_t)hi << 32) | lo;
}

// Descending sort of each wave's own PER * 64 composites (lane l holds
// wave positions l * PER + r) by a bitonic network in registers and lane
// exchanges.  In the merge of blocks of SIZE, position p keeps the larger
// value when bit STRIDE of p equals bit SIZE of p; with p = l * PER + r
// those are lane bits (or, below PER, bits of r), so each step's direction
// is a lane mask known at compile time, and SIZE = PER * 64 leaves every
// wave descending.  Templates, not loops, so that every step is unrolled.
template <int PER, int SIZE, int STRIDE>
__device__ __forceinline__ void wave_bitonic_step(uint64_t (&v)[PER])
{
    if constexpr (STRIDE < PER) {
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            if ((r & STRIDE) == 0) {
                const uint64_t hi = SIZE < PER ? ((r & SIZE) == 0 ? ~0ull : 0ull) : lanes_bit_clear(SIZE / PER);
                const uint64_t x = v[r], y = v[r + STRIDE];
                const bool t = take_first(hi, x, y);
                v[r] = t ? x : y;
                v[r + STRIDE] = t ? y : x;
            }
        }
    } else {
        constexpr int lx = STRIDE / PER;
        constexpr uint64_t hi = ~(lanes_bit_clear(lx) ^ lanes_bit_clear(SIZE / PER));
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const uint64_t y = lane_xor_u64(v[r], lx);
            v[r] = take_first(hi, v[r], y) ? v[r] : y;
        }
    }
    if constexpr (STRIDE > 1)
        wave_bitonic_step<PER, SIZE, STRIDE / 2>(v);
}

template <int PER, int SIZE = 2>
__device__ __forceinline__ void wave_bitonic_desc(uint64_t (&v)[PER])
{
    wave_bitonic_step<PER, SIZE, SIZE / 2>(v);
    if constexpr (SIZE < PER * kWave)
        wave_bitonic_desc<PER, SIZE * 2>(v);
}

// The m candidates in descending order of (key, -entry), the first k
// written (entries, -1 past m): each wave sorts PER * 64 of them, the sorted
// runs go to sb (PER * threads 64-bit words of LDS), and every candidate's
// final position is the number of composites above it, summed over the runs
// by a binary search in each.  Composites are distinct (entries are), so the
// positions are a permutation of 0 .. m-1.
template <int PER>
__device__ __forceinline__ void block_merge_write(const uint32_t *ckey, const uint32_t *cent, int m, int k,
                                                  uint64_t *sb, int32_t *out)
{
    constexpr int NW = kTopkBlockWaves, NT = NW * kWave, L = PER * kWave;
    const int t = threadIdx.x, wv = t / kWave;
    uint64_t v[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int p = t * PER + r;
        v[r] = p < m ? ((uint64_t)ckey[p] << 32) | (uint32_t)(0xFFFFFFFFu - cent[p]) : 0ull;
    }
    wave_bitonic_desc<PER>(v);
    __syncthreads(); // sb may overlap the candidate arrays
#pragma unroll
    for (int r = 0; r < PER; ++r)
        sb[t * PER + r] = v[r];
    __syncthreads();
    // a wave's candidates sort ahead of its zero padding, so position
    // t * PER + r holds a candidate exactly when it is below m
    if (wv * L < m) {
        int c[NW][PER];
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
            for (int r = 0; r < PER; ++r)
                c[w][r] = 0;
        // c = the largest count in [0, L-1] whose last composite is above v
#pragma unroll
        for (int st = L / 2; st > 0; st /= 2) {
            uint64_t a[NW][PER];
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
                for (int r = 0; r < PER; ++r)
                    a[w][r] = sb[w * L + c[w][r] + st - 1];
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
                for (int r = 0; r < PER; ++r)
                    c[w][r] += a[w][r] > v[r] ? st : 0;
        }
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            uint64_t a[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w)
                a[w] = sb[w * L + c[w][r]];
            int pos = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                pos += c[w][r] + (a[w] > v[r] ? 1 : 0);
            if (t * PER + r < m && pos < k)
                out[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)v[r]);
        }
    }
    for (int p = m + t; p < k; p += NT)
        out[p] = -1;
}

// Rows up to this length take the fast path: the row's keys fit in LDS.
constexpr int kTopkBlockFastMaxW = 32768;

// LDS of the fast path: the coarse histogram (later the candidates),
// the row's keys (later the sort buffer), the counters.
__host__ __device__ constexpr size_t topk_block_fast_lds_bytes(int W)
{
    return (size_t)kCoarseBins * 4 + (size_t)(W + 3) / 4 * 16 + 64;
}

__device__ __forceinline__ bool topk_block_fast(const float *src, int n, int k, unsigned char *smem, int32_t *out)
{
    constexpr int NW = kTopkBlockWaves, NT = NW * kWave, kB = 16;
    static_assert(2 * kBlockCandMax * 4 <= kCoarseBins * 4, "candidates fit the histogram's place");
    uint32_t *hist = reinterpret_cast<uint32_t *>(smem);
    uint32_t *ckey = hist, *cent = hist + kBlockCandMax;
    uint32_t *row = hist + kCoarseBins;
    const int n4 = (n + 3) / 4;
    int *part = reinterpret_cast<int *>(row + 4 * n4);
    const int t = threadIdx.x, wv = t / kWave;

    // pass 1: the keys to LDS and the coarse histogram; kB loads per thread
    // in flight (a 32768-entry row is one batch)
    coarse_clear<NW>(hist);
    __syncthreads();
    const bool vec = (reinterpret_cast<uintptr_t>(src) & 15u) == 0;
    const int nv = vec ? n / 4 : 0;
    const float4 *src4 = reinterpret_cast<const float4 *>(src);
    u32x4 *row4 = reinterpret_cast<u32x4 *>(row);
#pragma unroll 1
    for (int i0 = 0; i0 < nv; i0 += kB * NT) {
        float4 v[kB];
#pragma unroll
        for (int x = 0; x < kB; ++x) {
            const int i = i0 + x * NT + t;
            v[x] = i < nv ? src4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
#pragma unroll
        for (int x = 0; x < kB; ++x) {
            const int i = i0 + x * NT + t;
            const u32x4 kv = {score_key(v[x].x), score_key(v[x].y), score_key(v[x].z), score_key(v[x].w)};
            if (i < nv)
                row4[i] = kv;
            coarse_add(hist, kv.x);
            coarse_add(hist, kv.y);
            coarse_add(hist, kv.z);
            coarse_add(hist, kv.w);
        }
    }
    for (int j = nv * 4 + t; j < n; j += NT) {
        const uint32_t kv = score_key(src[j]);
        row[j] = kv;
        coarse_add(hist, kv);
    }
    __syncthreads();
    // candidates: the keys in [lo, kKeyPosInf]
    const int bin = coarse_find_bin<NW>(hist, k, part);
    uint32_t lo = coarse_tau(bin) + 1u;
    // this thread's keys: blocks i = t + NT x of four keys (entries past n
    // read as 0, never a candidate)
    auto block_keys = [&](int i) {
        u32x4 kv = row4[i];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * i + e >= n)
                kv[e] = 0u;
        return kv;
    };
    // pass 2 over the LDS row: find this thread's candidates (a bit per key:
    // its at most 16 blocks of four are 64 keys, the first 32 in hi32, the
    // rest in lo32, most significant bit first), place them by a workgroup
    // prefix sum (pos: this thread's first place, m: all candidates)
    static_assert(kTopkBlockFastMaxW <= 16 * 4 * NT, "64 keys per thread");
    uint32_t hi32, lo32;
    int pos, m;
    auto mark = [&]() {
        const uint32_t span = kKeyPosInf - lo;
        hi32 = 0u;
        lo32 = 0u;
#pragma unroll 4
        for (int i = t, x = 0; i < n4; i += NT, ++x) {
            const u32x4 kv = block_keys(i);
            uint32_t &wd = x < 8 ? hi32 : lo32;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                wd = 2u * wd + ((kv[e] - lo <= span) ? 1u : 0u);
        }
        // left-align the words of a thread with fewer than 16 blocks
        const int nx = (n4 - t + NT - 1) / NT; // blocks of this thread (t < n4), else <= 0
        if (nx < 8)
            hi32 = nx > 0 ? hi32 << (32 - 4 * nx) : 0u;
        else if (nx > 8 && nx < 16)
            lo32 = lo32 << (64 - 4 * nx);
        const int c = __builtin_popcount(hi32) + __builtin_popcount(lo32);
        const int incl = wave_inclusive_sum(c);
        if (lane() == kWave - 1)
            part[wv] = incl;
        __syncthreads();
        pos = incl - c;
        m = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            pos += w < wv ? part[w] : 0;
            m += part[w];
        }
    };
    mark();
    if (m > kBlockCandMax) {
        // The k-th largest key's bucket holds too many keys (ties, or scores
        // packed closely): histogram that bucket's keys by their next
        // kCoarseBits bits and move the threshold to the sub-bucket holding
        // the k-th largest key.
        if (bin < 0)
            return false; // fewer than k selectable keys: every one is a candidate
        const int above = m - (int)hist[bin];
        __syncthreads(); // hist[bin] and part read by every thread
        coarse_clear<NW>(hist);
        __syncthreads();
        constexpr int kSub = 32 - 2 * kCoarseBits;
        for (int i = t; i < n4; i += NT) {
            const u32x4 kv = block_keys(i);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (key_selectable(kv[e]) && (int)(kv[e] >> (32 - kCoarseBits)) == bin)
                    atomicAdd(&hist[(kv[e] >> kSub) & (kCoarseBins - 1)], 1u);
        }
        __syncthreads();
        const int sub = coarse_find_bin<NW>(hist, k - above, part);
        if (sub < 0)
            return false; // not reached: the bucket holds at least k - above keys
        lo = ((uint32_t)bin << (32 - kCoarseBits)) | ((uint32_t)sub << kSub);
        mark();
        if (m > kBlockCandMax)
            return false;
    }
    // key q (0 .. 63) of this thread is entry 4 (t + NT (q / 4)) + q % 4
    auto put = [&](uint32_t wd, int q0) {
        while (wd != 0u) {
            const int b = __builtin_clz(wd);
            wd &= ~(0x80000000u >> b);
            const int q = q0 + b;
            const uint32_t entry = (uint32_t)(4 * (t + NT * (q >> 2)) + (q & 3));
            ckey[pos] = row[entry];
            cent[pos] = entry;
            ++pos;
        }
    };
    put(hi32, 0);
    put(lo32, 32);
    __syncthreads();
    // the sort buffer takes the row's place: the LDS holds W >= 8192 keys on
    // this path, at least the 16 KB of 2048 composites (it may cover the
    // counters, which are not read again)
    uint64_t *sb = reinterpret_cast<uint64_t *>(row);
    if (m <= NT)
        block_merge_write<1>(ckey, cent, m, k, sb, out);
    else if (m <= 2 * NT)
        block_merge_write<2>(ckey, cent, m, k, sb, out);
    else
        block_merge_write<4>(ckey, cent, m, k, sb, out);
    return true;
}

__global__ __launch_bounds__(kTopkBlockWaves * kWave) void topk_block_kernel(const KernelArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int wv = uniform(threadIdx.x / kWave);
    const int64_t row = blockIdx.x;
    const int n = row_length(a, row);
    uint32_t *hist_all = reinterpret_cast<uint32_t *>(smem);            // [kTopkBlockWaves][256]
    uint32_t *keys = hist_all + kTopkBlockWaves * 256;                  // [kTopkBlockWaves][cap]
    uint32_t *ents = keys + (size_t)kTopkBlockWaves * a.cap;            // [kTopkBlockWaves][cap]
    int *cnt = reinterpret_cast<int *>(ents + (size_t)kTopkBlockWaves * a.cap);  // [kTopkBlockWaves + 2]
    uint32_t *sel_key = reinterpret_cast<uint32_t *>(cnt + kTopkBlockWaves + 2);  // [top_k]
    uint32_t *sel_ent = sel_key + a.top_k;                              // [top_k]
    // the coarse histogram reuses the wave buffers before they are filled
    static_assert(kCoarseBins <= kTopkBlockWaves * (256 + 2 * 576), "coarse histogram fits the buffers");
    // segments of whole 64-entry chunks
    const int chunks = (n + kWave - 1) / kWave;
    const int per = (chunks + kTopkBlockWaves - 1) / kTopkBlockWaves;
    const int j0 = min(wv * per * kWave, n), j1 = min((wv + 1) * per * kWave, n);
    const float *src = a.scores + row * a.W;
    // Rows whose keys fit in LDS (the workgroup has the LDS for W keys) take
    // the fast path unless it finds too many candidates.
    if (a.W <= kTopkBlockFastMaxW) {
        if (topk_block_fast(src, n, a.top_k, smem, a.idx + row * a.top_k))
            return;
        if (a.redo) { // the LDS holds the in-LDS path only: leave the row to topk_kernel
            if (threadIdx.x == 0)
                a.idx[row * a.top_k] = kTopkRedo;
            return;
        }
        __syncthreads(); // the streaming path below reuses the same LDS
    }
    TopKRow<uint32_t> tk;
    {
        const uint32_t tau0 = coarse_threshold<kTopkBlockWaves>(src, n, a.top_k, hist_all, cnt);
        topk_init(tk, keys + (size_t)wv * a.cap, ents + (size_t)wv * a.cap, hist_all + wv * 256, a.cap, a.top_k);
        tk.tau = tau0;
        if (j1 > j0)
            stream_row(tk, src, j0, j1, n);
    }

    // With the threshold preset the buffers usually end up holding a few
    // hundred pairs in all: gather them (segments in wave order, so entry
    // order) at the front and let one wave finish from registers.
    if (lane() == 0)
        cnt[wv] = tk.count;
    __syncthreads();
    int total = 0, before = 0;
#pragma unroll
    for (int w = 0; w < kTopkBlockWaves; ++w) {
        before += w < wv ? cnt[w] : 0;
        total += cnt[w];
    }
    if (total <= 24 * kWave && a.cap * kTopkBlockWaves >= 24 * kWave) {
        // two phases (read all, then write) since destinations overlap sources
        constexpr int kMaxPer = 24; // >= cap / 64 whenever total fits
        uint32_t kr[kMaxPer], er[kMaxPer];
        const int mine = tk.count;
#pragma unroll
        for (int r = 0; r < kMaxPer; ++r) {
            const int i = r * kWave + lane();
            kr[r] = i < mine ? tk.key[i] : 0u;
            er[r] = i < mine ? tk.ent[i] : 0u;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kMaxPer; ++r) {
            const int i = r * kWave + lane();
            if (i < mine) {
                keys[before + i] = kr[r];
                ents[before + i] = er[r];
            }
        }
        __syncthreads();
        if (wv == 0) {
            TopKRow<uint32_t> all;
            topk_init(all, keys, ents, hist_all, 24 * kWave, a.top_k);
            all.count = total;
            topk_finish_regs<24>(all, a.idx + row * a.top_k);
        }
        return;
    }
    topk_reduce(tk);
    block_select_sort<kTopkBlockWaves>(keys, ents, a.cap, tk.count, a.top_k, hist_all, cnt, sel_key, sel_ent,
                                       a.idx + row * a.top_k);
}

// ---------------------------------------------------------------------------
// KL divergence and its gradient from a dense score matrix: one workgroup per
// row.  Pass 1 folds the row's visible entries (finite scores; masked ones
// are -inf) into KL statistics, pass 2 overwrites each score with
// d kl / d score = exp(s - lse) - a / A (0 where masked, or when the row has
// no visible entry or no target mass).
// ---------------------------------------------------------------------------
constexpr int kKLGradWaves = 4;

__global__ __launch_bounds__(kKLGradWaves * kWave) void kl_grad_kernel(const KernelArgs a)
{
    __shared__ KLAcc part[kKLGradWaves];
    const int64_t row = blockIdx.x;
    const int wv = uniform(threadIdx.x / kWave);
    float *s = a.scores + row * a.W;
    const float *t = a.target + row * a.W;
    KLAcc acc = kl_empty();
    for (int j = threadIdx.x; j < a.W; j += kKLGradWaves * kWave) {
        const float sv = s[j];
        if (sv != -INFINITY)
            kl_add(acc, sv, t[j]);
    }
    acc = kl_wave_reduce(acc);
    if (lane() == 0)
        part[wv] = acc;
    __syncthreads();
    KLAcc tot = part[0];
#pragma unroll
    for (int w = 1; w < kKLGradWaves; ++w)
        tot = kl_merge(tot, part[w]);
    if (threadIdx.x == 0)
        a.kl[row] = kl_value(tot);
    const bool has = tot.m != -INFINITY && tot.A > 0.0f;
    const float lse = has ? tot.m + __logf(tot.se) : 0.0f;
    const float inv_a = has ? 1.0f / tot.A : 0.0f;
    for (int j = threadIdx.x; j < a.W; j += kKLGradWaves * kWave) {
        const float sv = s[j];
        s[j] = (has && sv != -INFINITY) ? __expf(sv - lse) - t[j] * inv_a : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------
size_t rows_lds_bytes(int D, int HB, int mode, int cap)
{
    size_t tile;
    if (HB <= 2) {
        switch (D) {
        case 32: tile = 2 * Tile3Geom<32>::kBufBytes; break;
        case 64: tile = 2 * Tile3Geom<64>::kBufBytes; break;
        default: tile = 2 * Tile3Geom<128>::kBufBytes; break;
        }
    } else {
        tile = 2 * (size_t)kTileEntries * (D + 8) * 2;
    }
    size_t sel = (mode & kModeSelect) ? (size_t)kRowWaves * rows_topk_wave_bytes(cap) : 0;
    return tile + sel;
}

size_t topk_lds_bytes(int cap) { return (size_t)kTopkWaves * (1024 + (size_t)cap * 8); }

size_t topk_block_fast_only_lds_bytes(int top_k, int W)
{
    // k close to the candidate room leaves the in-LDS path too little slack
    // to succeed on any row
    if (W < kTopkBlockMinLen || W > kTopkBlockFastMaxW || top_k > kBlockCandMax - kBlockCandMax / 16)
        return 0;
    return topk_block_fast_lds_bytes(W);
}

size_t topk_block_lds_bytes(int cap, int top_k, int W)
{
    const size_t stream = (size_t)kTopkBlockWaves * (1024 + (size_t)cap * 8) + (kTopkBlockWaves + 2) * 4 +
                          (size_t)top_k * 8;
    return W <= kTopkBlockFastMaxW ? max(stream, topk_block_fast_lds_bytes(W)) : stream;
}

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
    if constexpr (HB <= 2) {
        constexpr int G = kModeSegs;
        switch (mode | (a.k_seg ? G : 0)) {
        case kModeScores:
            return launch(rows3_kernel<D, HB, kModeScores>, grid, block, lds, s, a);
        case kModeSelect:
            return launch(rows3_kernel<D, HB, kModeSelect>, grid, block, lds, s, a);
        case kModeScores | kModeSelect:
            return launch(rows3_kernel<D, HB, kModeScores | kModeSelect>, grid, block, lds, s, a);
        case kModeKL:
            return launch(rows3_kernel<D, HB, kModeKL>, grid, block, lds, s, a);
        case kModeScores | G:
            return launch(rows3_kernel<D, HB, kModeScores | G>, grid, block, lds, s, a);
        case kModeSelect | G:
            return launch(rows3_kernel<D, HB, kModeSelect | G>, grid, block, lds, s, a);
        case kModeScores | kModeSelect | G:
            return launch(rows3_kernel<D, HB, kModeScores | kModeSelect | G>, grid, block, lds, s, a);
        case kModeKL | G:
            return launch(rows3_kernel<D, HB, kModeKL | G>, grid, block, lds, s, a);
        default:
            return hipErrorInvalidValue;
        }
    } else {
        switch (mode) {
        case kModeScores:
            return launch(rows_kernel<D, HB, kModeScores>, grid, block, lds, s, a);
        case kModeSelect:
            return launch(rows_kernel<D, HB, kModeSelect>, grid, block, lds, s, a);
        case kModeScores | kModeSelect:
            return launch(rows_kernel<D, HB, kModeScores | kModeSelect>, grid, block, lds, s, a);
        case kModeKL:
            return launch(rows_kernel<D, HB, kModeKL>, grid, block, lds, s, a);
        default:
            return hipErrorInvalidValue;
        }
    }
}

template <int D>
static hipError_t launch_rows_d(int HB, int mode, const KernelArgs &a, size_t lds, hipStream_t s)
{
    switch (HB) {
    case 1: return launch_rows_t<D, 1>(mode, a, lds, s);
    case 2: return launch_rows_t<D, 2>(mode, a, lds, s);
    case 4: return launch_rows_t<D, 4>(mode, a, lds, s);
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
    const size_t lds = (size_t)kSplitWaves * SplitGeom<D>::kWaveBytes;
    switch (HB) {
    case 1: return launch(split_kernel<D, 1>, grid, block, lds, s, a);
    case 2: return launch(split_kernel<D, 2>, grid, block, lds, s, a);
    case 4: return launch(split_kernel<D, 4>, grid, block, lds, s, a);
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

template <int D>
static hipError_t launch_stream_d(int HB, const KernelArgs &a, int blocks, hipStream_t s)
{
    dim3 grid((unsigned)blocks), block(kStreamWaves * kWave);
    const size_t lds = (size_t)kStreamWaves * SplitGeom<D>::kWaveBytes + (2 * kStreamSlots + 1) * sizeof(int);
    switch (HB) {
    case 1: return launch(stream_kernel<D, 1>, grid, block, lds, s, a);
    case 2: return launch(stream_kernel<D, 2>, grid, block, lds, s, a);
    case 4: return launch(stream_kernel<D, 4>, grid, block, lds, s, a);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_stream(int D, int HB, const KernelArgs &a, int blocks, hipStream_t s)
{
    if (a.rows > kStreamMaxRows)
        return hipErrorInvalidValue;
    switch (D) {
    case 32: return launch_stream_d<32>(HB, a, blocks, s);
    case 64: return launch_stream_d<64>(HB, a, blocks, s);
    case 128: return launch_stream_d<128>(HB, a, blocks, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_topk(const KernelArgs &a, size_t lds, hipStream_t s)
{
    dim3 grid((unsigned)((a.rows + kTopkWaves - 1) / kTopkWaves)), block(kTopkWaves * kWave);
    return launch(topk_kernel, grid, block, lds, s, a);
}

hipError_t launch_topk_block(const KernelArgs &a, size_t lds, hipStream_t s)
{
    dim3 grid((unsigned)a.rows), block(kTopkBlockWaves * kWave);
    return launch(topk_block_kernel, grid, block, lds, s, a);
}

hipError_t launch_kl_grad(const KernelArgs &a, hipStream_t s)
{
    dim3 grid((unsigned)a.rows), block(kKLGradWaves * kWave);
    return launch(kl_grad_kernel, grid, block, 0, s, a);
}

} // namespace csa
