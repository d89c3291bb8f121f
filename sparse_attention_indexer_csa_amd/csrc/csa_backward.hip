// Backward of the indexer score on MI355X (gfx950): the gradients of
// L = sum over unmasked (i, j) of g[b,i,j] * score[b,i,j] with respect to q, k
// and w, without the [B,H,S,W] per-head logits that differentiating the
// score through autodiff materialises (MaxText PR #5079 "Add StreamIndex
// Kernel for CSA", review of its custom VJP, which asks for a fused backward):
//
//   dw[b,i,h]   = scale * sum_j g[b,i,j] * ReLU(l)
//   dq[b,h,i,:] = scale * w[b,i,h] * sum_j g[b,i,j] * [l > 0] * k[b,j,:]
//   dk[b,j,:]   = scale * sum_i sum_h g[b,i,j] * w[b,i,h] * [l > 0] * q[b,h,i,:]
//
// with l = q[b,h,i,:] . k[b,j,:] recomputed per tile on MFMA exactly as the
// forward computes it.  Masked pairs take no part (a masked score is a
// constant).  The gradient operand of each product -- g [l>0] for dq,
// g w [l>0] for dk -- is rounded to bf16 once (round to nearest even) and
// contracted on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Pass 1 (bwd_rows_kernel): a workgroup owns a few query rows, one wave per
// (row, 32-head block); key tiles of 64 entries are staged in LDS and shared;
// the dq product reads its key operand down the tile's columns with
// transposing LDS reads.
// The transposed logits l[j, h] come out of the MFMA with one head per lane,
// which is the layout the dq product needs for its A operand, so the
// elementwise step stays in registers.  dw is a per-lane register sum.
// Pass 2 (bwd_keys_kernel): a workgroup owns 128 entries (one wave per 32) and
// a chunk of 256 rows; every row's q block and weights are staged in LDS and
// the logits l[h, j] come out with one entry per lane, the layout of the dk
// product's A operand.  Each (chunk, key tile) writes a partial to the
// workspace; pass 3 (bwd_reduce_kernel) sums the partials of every chunk that
// can see the tile, in chunk order, so results are deterministic.
#include "csa_backward.hpp"
#include "csa_score.hpp"

namespace csa {

namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * kWave;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (nearest, ties to even) and packed into one
// dword, lo in bits 0-15, hi in 16-31: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t cvt_pack_bf16(float lo, float hi)
{
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// MFMA operand from eight floats rounded to bf16 (k index e = element e).
__device__ __forceinline__ bf16x8 operand_from(const float (&v)[16], int base)
{
    u32x4 u;
    u.x = cvt_pack_bf16(v[base + 0], v[base + 1]);
    u.y = cvt_pack_bf16(v[base + 2], v[base + 3]);
    u.z = cvt_pack_bf16(v[base + 4], v[base + 5]);
    u.w = cvt_pack_bf16(v[base + 6], v[base + 7]);
    return __builtin_bit_cast(bf16x8, u);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Key tiles and q blocks sit in LDS row-major with D bf16 columns and no
// padding.  The 16-byte chunk c of row r is stored at chunk c ^ swizzle(r) of
// that row, so that with 64 four-byte banks neither access pattern conflicts:
// 16 lanes reading 16 consecutive rows at one chunk (row operands, staging
// stores), and a transposing read, whose 32 lanes read four consecutive rows
// at four consecutive chunks.  The swizzle uses bits 0-3 of the row only, and
// moving 8 rows down flips its bit 1.
template <int D>
__device__ __forceinline__ int swizzle(int r)
{
    static_assert(D == 32 || D == 64 || D == 128, "tile widths 32, 64, 128");
    if constexpr (D == 128)
        return 4 * (r & 3) + ((r >> 2) & 3);
    else if constexpr (D == 64)
        return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    else
        return (r >> 2) & 3;
}

// element offset of chunk c (columns 8c .. 8c+7) of row r
template <int D>
__device__ __forceinline__ int tile_offset(int r, int c)
{
    return r * D + 8 * (c ^ swizzle<D>(r));
}

// This lane's row operand addressing: row r (the lane's entry or head) at
// chunk 2s + gi (the eight values of k-step s) is at row_base + 8 * (2s ^ x).
struct RowLane {
    int row_base, x;
};

template <int D>
__device__ __forceinline__ RowLane row_lane(int r, int gi)
{
    return {r * D, gi ^ swizzle<D>(r)};
}

template <int D>
__device__ __forceinline__ bf16x8 load_row_operand(const uint16_t *tile, const RowLane &rl, int s)
{
    return load_frag(tile + rl.row_base + 8 * ((2 * s) ^ rl.x));
}

// An MFMA operand whose eight contraction values run down a column of a
// swizzled tile, read with two transposing LDS reads.  Within each 16-lane
// group, ds_read_b64_tr_b16 hands lane i element i % 4 of the 8-byte pieces
// addressed by lanes 4e + i / 4 (e = 0..3).  Lane l addresses row
// 4(l / 32) + (l / 4) % 4 of the block, columns 16((l / 16) % 2) + 4(l % 4) ..
// +3, and so receives rows c_row(0..7, l / 32) = {4g..4g+3, 8+4g..8+4g+3}
// (g = l / 32) of the 16-row block, column l % 32 of the 32-column block: the
// k layout of the operands produced from the 32x32 MFMA accumulators.
struct ColLane {
    int base, y;
};

template <int D>
__device__ __forceinline__ ColLane col_lane()
{
    const int l = lane();
    const int r = 4 * (l >> 5) + ((l >> 2) & 3);
    const int c = 2 * ((l >> 4) & 1) + ((l >> 1) & 1);
    return {r * D + 4 * (l & 1), c ^ swizzle<D>(r)};
}

// rows r0 .. r0+15 (r0 a multiple of 16), columns 32cb .. 32cb+31
template <int D>
__device__ __forceinline__ bf16x8 load_column_operand(const uint16_t *tile, const ColLane &cl, int r0, int cb)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const uint16_t *lo_p = tile + r0 * D + cl.base + 8 * ((4 * cb) ^ cl.y);
    const uint16_t *hi_p = tile + (r0 + 8) * D + cl.base + 8 * ((4 * cb) ^ cl.y ^ 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)lo_p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)hi_p);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ int64_t row_offset(const BwdArgs &a, int b)
{
    return a.q_offset ? (int64_t)a.q_offset[b] : 0;
}

// Whether any row of chunk c of batch b sees entry j0 (the first entry of a
// key tile).  Visibility grows with the row, so the chunk's last row decides.
// Both the key pass and the reduction use this, so a partial is read exactly
// when it was written.
__device__ __forceinline__ bool chunk_live(const BwdArgs &a, int b, int c, int j0)
{
    const int last = min((c + 1) * kBwdChunkRows, a.S) - 1;
    return visible_entries(row_offset(a, b) + last, a.m, a.W) > j0;
}

// ---------------------------------------------------------------------------
// Pass 1: dq and dw.

// Entries per key tile of the row pass: two 32-entry subtiles between
// barriers.
constexpr int kRowTile = 64;

template <int D>
struct RowTileGeom {
    static constexpr int kChunks = kRowTile * D / 8;      // 16-byte pieces per key tile
    static constexpr int kPerThread = (kChunks + kBwdThreads - 1) / kBwdThreads;
};

template <int D, int HB>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void bwd_rows_kernel(const BwdArgs a)
{
    using G = RowTileGeom<D>;
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int RPW = kBwdWaves / HB; // query rows per workgroup
    // key tile, entry-major and swizzled: A operand of the logits by 16-byte
    // reads, B operand of the dq product by transposing reads
    __shared__ __attribute__((aligned(16))) uint16_t tile[2][kRowTile * D];
    // each row's upstream gradients of the tile, 0 where masked
    __shared__ __attribute__((aligned(16))) float gtile[2][RPW][kRowTile];

    const int tid = threadIdx.x;
    const int wv = uniform(tid / kWave);
    const int l = lane(), n = l & 31, gi = l >> 5;
    const int hb = wv % HB;
    const int nrb = (a.S + RPW - 1) / RPW;
    const int b = blockIdx.x / nrb;
    // longest rows first
    const int i0 = (nrb - 1 - (int)(blockIdx.x % nrb)) * RPW;
    const int i = i0 + wv / HB;
    const bool active = i < a.S;
    const int64_t off = row_offset(a, b);
    const int last = min(i0 + RPW, a.S) - 1;
    const int ntiles = (visible_entries(off + last, a.m, a.W) + kRowTile - 1) / kRowTile;
    const int thr = active ? visible_entries(off + i, a.m, a.W) : 0;
    const int qseg = (active && a.q_seg) ? a.q_seg[(int64_t)b * a.S + i] : 0;

    // B operand of the transposed logits: this lane's head (32hb + n), eight
    // values of D per k-step.  Heads past H read head H-1 (never written out).
    bf16x8 qf[KS];
    if (active) {
        const uint16_t *qp = a.q + (int64_t)b * a.q_sb + (int64_t)min(32 * hb + n, a.H - 1) * a.q_sh +
                             (int64_t)i * a.q_ss + 8 * gi;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qf[s] = load_frag(qp + 16 * s);
    } else {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qf[s] = zero_frag();
    }
    const float *grow = a.g + ((int64_t)b * a.S + (active ? i : 0)) * a.W;
    const uint16_t *kb = a.k + (int64_t)b * a.k_sb;

    f32x16 acc[DB];
#pragma unroll
    for (int c = 0; c < DB; ++c)
        for (int r = 0; r < 16; ++r)
            acc[c][r] = 0.0f;
    float dw_acc = 0.0f;

    // this lane's addressing of the key tile: entry n of a 32-entry subtile
    // (logits), entries c_row(0..7, gi) of a 16-entry block, column n (dq)
    const RowLane krow = row_lane<D>(n, gi);
    const ColLane kcol = col_lane<D>();
    // Staging: piece c holds eight columns 8(c / kRowTile) .. +7 of entry
    // c % kRowTile, so the lanes of a wave cover consecutive entries.
    uint4 pre[G::kPerThread];
    auto fetch = [&](int t) {
#pragma unroll
        for (int u = 0; u < G::kPerThread; ++u) {
            const int c = tid + u * kBwdThreads;
            const int row = c % kRowTile, col = (c / kRowTile) * 8;
            const int j = kRowTile * t + row;
            pre[u] = make_uint4(0, 0, 0, 0);
            if (c < G::kChunks && j < a.W)
                pre[u] = *reinterpret_cast<const uint4 *>(kb + (int64_t)j * a.k_sw + col);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int u = 0; u < G::kPerThread; ++u) {
            const int c = tid + u * kBwdThreads;
            const int row = c % kRowTile, col = (c / kRowTile) * 8;
            if (c < G::kChunks)
                *reinterpret_cast<uint4 *>(&tile[buf][tile_offset<D>(row, col / 8)]) = pre[u];
        }
    };

    // The masked gradients of a row's tile are loaded once, by the row's
    // first head-block wave (one entry per lane), and staged in LDS with the
    // key tile.  The loaded values are masked only when they are stored, after
    // the tile's products: using them earlier would make the wave wait for the
    // loads before its matrix work.
    static_assert(kRowTile == kWave, "one gradient per lane");
    const int wr = wv / HB; // this wave's row within the workgroup
    const bool g_lane = hb == 0;
    float gnext = 0.0f; // gradient of this lane's next entry, as loaded
    int snext = 0;      // its segment id, as loaded
    bool gvis = false;  // whether the entry is before the row's threshold
    auto fetch_g = [&](int t) {
        if (g_lane && active) {
            const int j = kRowTile * t + l;
            const int jc = min(j, a.W - 1);
            gvis = j < thr;
            if (a.k_seg)
                snext = a.k_seg[(int64_t)b * a.W + jc];
            gnext = grow[jc];
        }
    };
    auto store_g = [&](int buf) {
        if (g_lane) {
            const bool ok = gvis && (!a.k_seg || snext == qseg);
            gtile[buf][wr][l] = ok ? gnext : 0.0f;
        }
    };

    if (ntiles > 0) {
        fetch(0);
        fetch_g(0);
        store(0);
        store_g(0);
    }
    // Every load issued so far (the q operands included) completes here, so
    // that inside the loop only the next tile's loads are in flight and the
    // products never wait for them.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) {
            fetch(t + 1);
            fetch_g(t + 1);
        }
#pragma unroll
        for (int hs = 0; hs < kRowTile / 32; ++hs) {
        if (active && kRowTile * t + 32 * hs < thr) {
            const uint16_t *T = tile[t & 1] + 32 * hs * D;
            // upstream gradient of this lane's 16 entries c_row(r, gi)
            float ge[16];
            const float *gt = gtile[t & 1][wr] + 32 * hs;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 v = *reinterpret_cast<const float4 *>(gt + 8 * q4 + 4 * gi);
                ge[4 * q4 + 0] = v.x;
                ge[4 * q4 + 1] = v.y;
                ge[4 * q4 + 2] = v.z;
                ge[4 * q4 + 3] = v.w;
            }
            // transposed logits: lane = head n of this block, register r = entry c_row(r, gi)
            f32x16 lt;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                lt[r] = 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                lt = mfma32(load_row_operand<D>(T, krow, s), qf[s], lt);
            float pf[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float x = lt[r];
                dw_acc = fmaf(ge[r], relu(x), dw_acc);
                pf[r] = x > 0.0f ? ge[r] : 0.0f; // rounded to bf16 by operand_from
            }
            const bf16x8 a0 = operand_from(pf, 0), a1 = operand_from(pf, 8);
            // B operand: entries 32hs + c_row(0..7, gi) (+16), column 32c + n
#pragma unroll
            for (int c = 0; c < DB; ++c) {
                acc[c] = mfma32(a0, load_column_operand<D>(T, kcol, 0, c), acc[c]);
                acc[c] = mfma32(a1, load_column_operand<D>(T, kcol, 16, c), acc[c]);
            }
        }
        }
        if (t + 1 < ntiles) {
            store((t + 1) & 1);
            store_g((t + 1) & 1);
        }
        __syncthreads();
    }

    // lanes n and n + 32 hold the same head over different entries
    const float dw_sum = dw_acc + __shfl_xor(dw_acc, 32);
    if (!active)
        return;
    const int hd = 32 * hb + n;
    if (gi == 0 && hd < a.H)
        a.dw[((int64_t)b * a.S + i) * a.H + hd] = a.scale * dw_sum;
    // the weights of this lane's 16 heads, all loaded before the first store
    // (a store in between would keep each load waiting on the previous one)
    const uint16_t *wrow = a.w + (int64_t)b * a.w_sb + (int64_t)i * a.w_ss;
    uint16_t wh[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        wh[r] = wrow[min(32 * hb + c_row(r, gi), a.H - 1)];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int h = 32 * hb + c_row(r, gi);
        if (h < a.H) {
            const float f = a.scale * bf16_to_f32(wh[r]);
            float *dst = a.dq + (((int64_t)b * a.H + h) * a.S + i) * D + n;
#pragma unroll
            for (int c = 0; c < DB; ++c)
                dst[32 * c] = f * acc[c][r];
        }
    }
}

// ---------------------------------------------------------------------------
// Pass 2: per-chunk partial key gradients.

template <int D, int HB>
struct KeyGeom {
    static constexpr int kHeads = 32 * HB;
    static constexpr int kChunks = kHeads * D / 8; // 16-byte pieces of one row's q block
    static constexpr int kPerThread = (kChunks + kBwdThreads - 1) / kBwdThreads;
    static constexpr size_t kQBytes = (size_t)kHeads * D * 2;
    static constexpr size_t kLdsBytes = 2 * kQBytes + 2 * (size_t)kHeads * 4;
};

template <int D, int HB>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void bwd_keys_kernel(const BwdArgs a)
{
    using G = KeyGeom<D, HB>;
    constexpr int KS = D / 16, DB = D / 32, NH = G::kHeads;
    extern __shared__ __attribute__((aligned(16))) unsigned char bwd_smem[];
    // two buffers of one row's q block [NH][D] bf16 (swizzled), then two of
    // its weights [NH] fp32
    auto qbuf = [&](int buf) { return reinterpret_cast<uint16_t *>(bwd_smem + buf * G::kQBytes); };
    auto wbuf = [&](int buf) { return reinterpret_cast<float *>(bwd_smem + 2 * G::kQBytes + buf * NH * 4); };

    // Workgroup -> (batch, chunk, key tile).  Workgroups are dealt to the 8
    // XCDs in turn; XCD x takes every 8th chunk (latest rows first) with all
    // of its key tiles in a row, so the tiles of one chunk run side by side on
    // one XCD and share its L2 copy of the chunk's q rows.
    const int per_b = 8 * ((a.n_chunks + 7) / 8) * a.n_jtiles;
    const int b = blockIdx.x / per_b;
    const int r_ = blockIdx.x % per_b;
    const int x = r_ % 8, k_ = r_ / 8;
    const int chunk = a.n_chunks - 1 - (8 * (k_ / a.n_jtiles) + x);
    const int jt = k_ % a.n_jtiles;
    if (chunk < 0)
        return;
    const int j0 = jt * kBwdKeyTile;
    if (!chunk_live(a, b, chunk, j0))
        return;
    const int64_t off = row_offset(a, b);
    const int c0 = chunk * kBwdChunkRows, c1 = min(c0 + kBwdChunkRows, a.S);
    // first row that sees entry j0: (off + i + 1) div m > j0
    const int64_t i_min = ((int64_t)j0 + 1) * a.m - 1 - off;
    const int i_lo = (int)max((int64_t)c0, i_min);

    const int tid = threadIdx.x;
    const int wv = uniform(tid / kWave);
    const int l = lane(), n = l & 31, gi = l >> 5;
    const int jw = j0 + 32 * wv; // this wave's first entry
    const int j = jw + n;        // this lane's entry (logit column, dk A row)
    const bool wave_has = jw < a.W;

    // B operand of the logits: this lane's entry, eight values of D per k-step.
    bf16x8 kf[KS];
    {
        const uint16_t *kp = a.k + (int64_t)b * a.k_sb + (int64_t)min(j, a.W - 1) * a.k_sw + 8 * gi;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kf[s] = j < a.W ? load_frag(kp + 16 * s) : zero_frag();
    }
    const int kseg = a.k_seg ? a.k_seg[(int64_t)b * a.W + min(j, a.W - 1)] : 0;

    // this lane's addressing of the q block: head n of a 32-head block
    // (logits), heads c_row(0..7, gi) of a 16-head block, column n (dk)
    const RowLane qrow = row_lane<D>(n, gi);
    const ColLane qcol = col_lane<D>();

    f32x16 acc[DB];
#pragma unroll
    for (int c = 0; c < DB; ++c)
        for (int r = 0; r < 16; ++r)
            acc[c][r] = 0.0f;

    // Staging of the next row: its q block and weights (as loaded, converted
    // when stored) and this lane's gradient and segment id, which the row's
    // iteration copies before the next loads are issued, so that no loaded
    // value is used before the products that follow the loads.
    uint4 pre[G::kPerThread];
    uint16_t wraw = 0;
    float gnext = 0.0f;
    int snext = 0;
    auto fetch = [&](int i) {
        const uint16_t *qrow = a.q + (int64_t)b * a.q_sb + (int64_t)i * a.q_ss;
#pragma unroll
        for (int u = 0; u < G::kPerThread; ++u) {
            const int c = tid + u * kBwdThreads;
            const int h = c / (D / 8), col = (c % (D / 8)) * 8;
            pre[u] = make_uint4(0, 0, 0, 0);
            if (c < G::kChunks && h < a.H)
                pre[u] = *reinterpret_cast<const uint4 *>(qrow + (int64_t)h * a.q_sh + col);
        }
        if (tid < NH && tid < a.H)
            wraw = a.w[(int64_t)b * a.w_sb + (int64_t)i * a.w_ss + tid];
        gnext = a.g[((int64_t)b * a.S + i) * a.W + min(j, a.W - 1)];
        if (a.q_seg)
            snext = a.q_seg[(int64_t)b * a.S + i];
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int u = 0; u < G::kPerThread; ++u) {
            const int c = tid + u * kBwdThreads;
            const int h = c / (D / 8), col = (c % (D / 8)) * 8;
            if (c < G::kChunks)
                *reinterpret_cast<uint4 *>(qbuf(buf) + tile_offset<D>(h, col / 8)) = pre[u];
        }
        if (tid < NH)
            wbuf(buf)[tid] = bf16_to_f32(wraw); // heads past H: 0
    };

    fetch(i_lo);
    store(0);
    // Every load issued so far completes here (see the row pass).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = i_lo; i < c1; ++i) {
        const int buf = (i - i_lo) & 1;
        const float g_i = gnext;
        const int s_i = snext;
        if (i + 1 < c1)
            fetch(i + 1);
        const int thr = visible_entries(off + i, a.m, a.W);
        bool ok = j < thr;
        if (a.k_seg)
            ok = ok && kseg == s_i;
        const float ge = ok ? g_i : 0.0f;
        if (wave_has && ballot(ok) != 0) {
            const uint16_t *Q = qbuf(buf);
            const float *Wt = wbuf(buf);
            // rolled for two head blocks (fewer live registers), unrolled for four
            constexpr int kHbUnroll = HB == 4 ? 4 : 1;
#pragma unroll kHbUnroll
            for (int hb = 0; hb < HB; ++hb) {
                const uint16_t *Qh = Q + 32 * hb * D;
                // logits: lane = entry n, register r = head 32hb + c_row(r, gi)
                f32x16 lg;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    lg[r] = 0.0f;
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    lg = mfma32(load_row_operand<D>(Qh, qrow, s), kf[s], lg);
                float pf[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    // c_row(4 q4 + c, gi) = 8 q4 + 4 gi + c: four consecutive heads
                    const float4 wq = *reinterpret_cast<const float4 *>(Wt + 32 * hb + 8 * q4 + 4 * gi);
                    const float wr[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int r = 4 * q4 + c;
                        pf[r] = lg[r] > 0.0f ? ge * wr[c] : 0.0f; // rounded to bf16 by operand_from
                    }
                }
                const bf16x8 a0 = operand_from(pf, 0), a1 = operand_from(pf, 8);
#pragma unroll
                for (int c = 0; c < DB; ++c) {
                    acc[c] = mfma32(a0, load_column_operand<D>(Qh, qcol, 0, c), acc[c]);
                    acc[c] = mfma32(a1, load_column_operand<D>(Qh, qcol, 16, c), acc[c]);
                }
            }
        }
        if (i + 1 < c1)
            store(buf ^ 1);
        __syncthreads();
    }

    // partial[b, chunk, entry, d]: lane = column 32c + n, register r = entry jw + c_row(r, gi)
    float *dst = a.part + (((int64_t)b * a.n_chunks + chunk) * a.W) * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int je = jw + c_row(r, gi);
        if (je < a.W) {
#pragma unroll
            for (int c = 0; c < DB; ++c)
                dst[(int64_t)je * D + 32 * c + n] = acc[c][r];
        }
    }
}

// ---------------------------------------------------------------------------
// Pass 3: dk = scale * (sum of the live chunks' partials, in chunk order).

__global__ __launch_bounds__(256) void bwd_reduce_kernel(const BwdArgs a)
{
    const int D = a.D;
    const int64_t per_b = (int64_t)a.W * D / 4;
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= (int64_t)a.B * per_b)
        return;
    const int b = (int)(v / per_b);
    const int64_t e = (v % per_b) * 4; // element within [W, D]
    const int jtile0 = (int)(e / D) / kBwdKeyTile * kBwdKeyTile;
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int c = 0; c < a.n_chunks; ++c) {
        if (!chunk_live(a, b, c, jtile0))
            continue;
        const float4 p = *reinterpret_cast<const float4 *>(a.part + (((int64_t)b * a.n_chunks + c) * a.W) * D + e);
        s.x += p.x;
        s.y += p.y;
        s.z += p.z;
        s.w += p.w;
    }
    float4 o = make_float4(a.scale * s.x, a.scale * s.y, a.scale * s.z, a.scale * s.w);
    *reinterpret_cast<float4 *>(a.dk + (int64_t)b * a.W * D + e) = o;
}

template <int D, int HB>
hipError_t launch_rows_t(const BwdArgs &a, hipStream_t s)
{
    constexpr int RPW = kBwdWaves / HB;
    const int64_t blocks = (int64_t)a.B * ((a.S + RPW - 1) / RPW);
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL((bwd_rows_kernel<D, HB>), dim3((unsigned)blocks), dim3(kBwdThreads), 0, s, a);
    return hipGetLastError();
}

template <int D, int HB>
hipError_t launch_keys_t(const BwdArgs &a, hipStream_t s)
{
    const int64_t blocks = (int64_t)a.B * 8 * ((a.n_chunks + 7) / 8) * a.n_jtiles;
    if (blocks == 0)
        return hipSuccess;
    const size_t lds = KeyGeom<D, HB>::kLdsBytes;
    auto kernel = bwd_keys_kernel<D, HB>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kBwdThreads), lds, s, a);
    return hipGetLastError();
}

} // namespace

#define CSA_BWD_DISPATCH(FN, D, HB, ...)                                                                     \
    switch ((D) * 10 + (HB)) {                                                                               \
    case 321: return FN<32, 1>(__VA_ARGS__);                                                                 \
    case 322: return FN<32, 2>(__VA_ARGS__);                                                                 \
    case 324: return FN<32, 4>(__VA_ARGS__);                                                                 \
    case 641: return FN<64, 1>(__VA_ARGS__);                                                                 \
    case 642: return FN<64, 2>(__VA_ARGS__);                                                                 \
    case 644: return FN<64, 4>(__VA_ARGS__);                                                                 \
    case 1281: return FN<128, 1>(__VA_ARGS__);                                                               \
    case 1282: return FN<128, 2>(__VA_ARGS__);                                                               \
    case 1284: return FN<128, 4>(__VA_ARGS__);                                                               \
    default: return hipErrorInvalidValue;                                                                    \
    }

hipError_t launch_bwd_rows(int D, int HB, const BwdArgs &a, hipStream_t s)
{
    CSA_BWD_DISPATCH(launch_rows_t, D, HB, a, s)
}

hipError_t launch_bwd_keys(int D, int HB, const BwdArgs &a, hipStream_t s)
{
    CSA_BWD_DISPATCH(launch_keys_t, D, HB, a, s)
}

hipError_t launch_bwd_reduce(const BwdArgs &a, hipStream_t s)
{
    const int64_t n = (int64_t)a.B * a.W * a.D / 4;
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace csa
