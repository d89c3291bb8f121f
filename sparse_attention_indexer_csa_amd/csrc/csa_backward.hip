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

// The staging lambdas capture register arrays by reference: one left out of
// line would move those arrays to scratch memory.
#define CSA_INLINE __attribute__((always_inline))

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

// bits = 2 * bits + (bit of this lane in mask): one v_addc_co_u32 with the
// lane mask of a comparison as its carry-in (the compiler's own lowering of
// that expression takes two or three instructions per bit).
__device__ __forceinline__ void shift_in(uint32_t &bits, uint64_t mask)
{
    asm("v_addc_co_u32 %0, vcc, %0, %0, %1" : "+v"(bits) : "s"(mask) : "vcc");
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
    // logit-sign words of this row and this lane's head, as 16-bit halves
    const bool n_head_ok = active && 32 * hb + n < a.H;
    uint16_t *sign_row = reinterpret_cast<uint16_t *>(a.sign) +
                         (((int64_t)b * a.S + (active ? i : 0)) * a.n_blk * a.H + 32 * hb + n) * 2;

    // this lane's addressing of the key tile: entry n of a 32-entry subtile
    // (logits), entries c_row(0..7, gi) of a 16-entry block, column n (dq)
    const RowLane krow = row_lane<D>(n, gi);
    const ColLane kcol = col_lane<D>();
    // Staging: piece c holds eight columns 8(c / kRowTile) .. +7 of entry
    // c % kRowTile, so the lanes of a wave cover consecutive entries.  Entries
    // past W repeat entry W - 1 (their gradient is zero; every entry of k
    // below W must be finite).  The loads are unconditional, so that the waits
    // for them are the same on every path: the tile after the last one
    // repeats the last one and is never read.
    u32x4 pre[G::kPerThread]; // a vector type: HIP's uint4 struct is copied through memory
    int k_off[G::kPerThread]; // row * k_sw + col (< 2^30: k_sw < 2^24)
#pragma unroll
    for (int u = 0; u < G::kPerThread; ++u) {
        const int c = min(tid + u * kBwdThreads, G::kChunks - 1);
        k_off[u] = (c % kRowTile) * (int)a.k_sw + (c / kRowTile) * 8;
    }
    auto fetch = [&](int t) CSA_INLINE {
        if (kRowTile * (t + 1) <= a.W) {
            const uint16_t *kt = kb + (int64_t)kRowTile * t * a.k_sw;
#pragma unroll
            for (int u = 0; u < G::kPerThread; ++u)
                pre[u] = *reinterpret_cast<const u32x4 *>(kt + k_off[u]);
        } else {
#pragma unroll
            for (int u = 0; u < G::kPerThread; ++u) {
                const int c = min(tid + u * kBwdThreads, G::kChunks - 1);
                const int j = min(kRowTile * t + c % kRowTile, a.W - 1);
                pre[u] = *reinterpret_cast<const u32x4 *>(kb + (int64_t)j * a.k_sw + (c / kRowTile) * 8);
            }
        }
    };
    auto store = [&](int buf) CSA_INLINE {
#pragma unroll
        for (int u = 0; u < G::kPerThread; ++u) {
            const int c = tid + u * kBwdThreads;
            const int row = c % kRowTile, col = (c / kRowTile) * 8;
            if (c < G::kChunks)
                *reinterpret_cast<u32x4 *>(&tile[buf][tile_offset<D>(row, col / 8)]) = pre[u];
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
    auto fetch_g = [&](int t) CSA_INLINE {
        if (g_lane && active) {
            const int j = kRowTile * t + l;
            const int jc = min(j, a.W - 1);
            gvis = j < thr;
            if (a.k_seg)
                snext = a.k_seg[(int64_t)b * a.W + jc];
            gnext = grow[jc];
        }
    };
    auto store_g = [&](int buf) CSA_INLINE {
        if (g_lane) {
            const bool ok = gvis && (!a.k_seg || snext == qseg);
            gtile[buf][wr][l] = ok ? gnext : 0.0f;
        }
    };

    // One key tile; P = t % 2 selects the LDS buffers, so that every LDS
    // address is a lane offset plus a constant.
    auto tile_step = [&](int t, auto P_) CSA_INLINE {
        constexpr int P = decltype(P_)::value;
        const int tn = min(t + 1, ntiles - 1);
        fetch(tn);
        fetch_g(tn);
#pragma unroll
        for (int hs = 0; hs < kRowTile / 32; ++hs) {
            if (active && kRowTile * t + 32 * hs < thr) {
                const uint16_t *T = tile[P] + 32 * hs * D;
                // upstream gradient of this lane's 16 entries c_row(r, gi)
                float ge[16];
                const float *gt = gtile[P][wr] + 32 * hs;
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
                uint32_t sbits = 0; // bit 15 - r: [l > 0] of entry c_row(r, gi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = lt[r];
                    pf[r] = x > 0.0f ? ge[r] : 0.0f; // rounded to bf16 by operand_from
                    // g ReLU(x) accumulated as (g [x > 0]) x: the same value
                    // for finite x (x <= 0 adds a zero), one instruction fewer
                    dw_acc = fmaf(pf[r], x, dw_acc);
                    shift_in(sbits, ballot(x > 0.0f));
                }
                // the signs go to the key pass: this lane's half (16 bits) of the
                // word of head 32hb + n and the subtile's 32-entry block
                if (n_head_ok)
                    sign_row[(int64_t)(2 * t + hs) * a.H * 2 + gi] = (uint16_t)sbits;
                const bf16x8 a0 = operand_from(pf, 0), a1 = operand_from(pf, 8);
                // B operand: entries 32hs + c_row(0..7, gi) (+16), column 32c + n;
                // column block c + 1 is read while block c's products run
                // (kept in that order by scheduling barriers)
                bf16x8 b0 = load_column_operand<D>(T, kcol, 0, 0), b1 = load_column_operand<D>(T, kcol, 16, 0);
#pragma unroll
                for (int c = 0; c < DB; ++c) {
                    bf16x8 n0 = b0, n1 = b1;
                    if (c + 1 < DB) {
                        n0 = load_column_operand<D>(T, kcol, 0, c + 1);
                        n1 = load_column_operand<D>(T, kcol, 16, c + 1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    acc[c] = mfma32(a0, b0, acc[c]);
                    acc[c] = mfma32(a1, b1, acc[c]);
                    __builtin_amdgcn_sched_barrier(0);
                    b0 = n0;
                    b1 = n1;
                }
            }
        }
        store(P ^ 1); // after the last tile: stored, never read
        store_g(P ^ 1);
        __syncthreads();
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
    for (int t = 0; t < ntiles; t += 2) {
        tile_step(t, std::integral_constant<int, 0>());
        if (t + 1 < ntiles)
            tile_step(t + 1, std::integral_constant<int, 1>());
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
    static constexpr int kBlocks = kBwdKeyTile / 32;  // 32-entry blocks of a key tile (one per wave)
    static constexpr int kSignWords = kBlocks * kHeads; // sign words of one row and one key tile
    static constexpr int kSignPerThread = (kSignWords + kBwdThreads - 1) / kBwdThreads;
    static constexpr size_t kQBytes = (size_t)kHeads * D * 2;
    static constexpr size_t kWBytes = (size_t)kHeads * 4;
    static constexpr size_t kSBytes = (size_t)kSignWords * 4;
    // Rows staged three deep, except with four head blocks, where three
    // buffers of the 32 KB q block would leave one workgroup per compute unit.
    static constexpr int kDeep = HB <= 2 ? 3 : 2;
    static constexpr size_t kLdsBytes = kDeep * (kQBytes + kWBytes + kSBytes);
};

// Position, in a sign word, of the bit of entry e (0..31) of its block: the
// row pass writes the 16 bits of entries c_row(0..15, g) of lane half g as
// bits 16g + 15 - r.
__device__ __forceinline__ int sign_bit_of_entry(int e)
{
    const int g = (e >> 2) & 1, r = 4 * (e >> 3) + (e & 3); // e = c_row(r, g)
    return 16 * g + 15 - r;
}

template <int D, int HB>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(HB == 4 ? 2 : 3))) void bwd_keys_kernel(const BwdArgs a)
{
    using G = KeyGeom<D, HB>;
    constexpr int DB = D / 32, NH = G::kHeads;
    static_assert(G::kBlocks == kBwdWaves, "one 32-entry block per wave");
    extern __shared__ __attribute__((aligned(16))) unsigned char bwd_smem[];
    // kDeep buffers each of one row's q block [NH][D] bf16 (swizzled), its
    // weights [NH] fp32 and its sign words [kBlocks][NH]
    auto qbuf = [&](int buf) { return reinterpret_cast<uint16_t *>(bwd_smem + buf * G::kQBytes); };
    auto wbuf = [&](int buf) {
        return reinterpret_cast<float *>(bwd_smem + G::kDeep * G::kQBytes + buf * G::kWBytes);
    };
    auto sbuf = [&](int buf) {
        return reinterpret_cast<uint32_t *>(bwd_smem + G::kDeep * (G::kQBytes + G::kWBytes) + buf * G::kSBytes);
    };

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
    const int j = jw + n;        // this lane's entry (dk A row)
    const bool wave_has = jw < a.W;
    const int kseg = a.k_seg ? a.k_seg[(int64_t)b * a.W + min(j, a.W - 1)] : 0;
    const int sbit = sign_bit_of_entry(n);

    // this lane's addressing of the q block: heads c_row(0..7, gi) of a
    // 16-head block, column n
    const ColLane qcol = col_lane<D>();

    f32x16 acc[DB];
#pragma unroll
    for (int c = 0; c < DB; ++c)
        for (int r = 0; r < 16; ++r)
            acc[c][r] = 0.0f;

    // Staging, three rows deep.  Row r's q block, weights and sign words sit
    // in LDS buffer (r - i_lo) % 3 from the end of row r - 2 on, so that while
    // row i's products run, the A operand of row i + 1's first head block is
    // built from its buffer.  The q block and the weights of row i + 2
    // (shared by every key tile of the chunk, so mostly L2 hits) are loaded
    // during row i; the sign words, this lane's gradient and the row's
    // segment id (read once, from HBM) three rows ahead, in three register
    // slots indexed like the buffers.  No loaded value is used before the
    // products that follow its load: the loads are unconditional (clamped
    // addresses) and what lies outside the problem is zeroed when stored,
    // the weights are converted when stored, and a slot is read before the
    // next load into it is issued.  The far loads are issued after the q
    // block's, so that waiting for the q block leaves them in flight.
    // The row addresses advance by one row's stride per step (wave-uniform
    // pointer bumps, no 64-bit index products in the loop), and so do the
    // causal thresholds (no division in the loop).
    u32x4 pre[G::kPerThread]; // a vector type: HIP's uint4 struct is copied through memory
    uint16_t wraw = 0;
    uint32_t sgn[3][G::kSignPerThread];
    float gsl[3] = {0.0f, 0.0f, 0.0f};
    int ssl[3] = {0, 0, 0};
    const int blk0 = j0 / 32;
    // per-thread offsets within a row (loop invariant)
    int64_t q_off[G::kPerThread];
#pragma unroll
    for (int u = 0; u < G::kPerThread; ++u) {
        const int c = min(tid + u * kBwdThreads, G::kChunks - 1);
        q_off[u] = (int64_t)min(c / (D / 8), a.H - 1) * a.q_sh + (c % (D / 8)) * 8;
    }
    int s_off[G::kSignPerThread];
#pragma unroll
    for (int u = 0; u < G::kSignPerThread; ++u) {
        const int c = tid + u * kBwdThreads;
        s_off[u] = min(blk0 + c / NH, a.n_blk - 1) * a.H + min(c % NH, a.H - 1);
    }
    const int g_off = min(j, a.W - 1);
    const bool w_lane = tid < NH && tid < a.H;
    // near rows (q block, weights) and far rows (signs, gradient, segment id)
    const int64_t bs = (int64_t)b * a.S;
    const uint16_t *q_row = a.q + (int64_t)b * a.q_sb + (int64_t)i_lo * a.q_ss;
    const uint16_t *w_row = a.w + (int64_t)b * a.w_sb + (int64_t)i_lo * a.w_ss;
    const uint32_t *s_row = a.sign + (bs + i_lo) * a.n_blk * a.H;
    const float *g_row = a.g + (bs + i_lo) * a.W;
    // without segments the first word of g is read instead and never used
    // (the load is unconditional like the others)
    const int32_t *seg_row = a.q_seg ? a.q_seg + bs + i_lo : reinterpret_cast<const int32_t *>(a.g);
    const int64_t s_stride = (int64_t)a.n_blk * a.H;
    const int seg_stride = a.q_seg ? 1 : 0;
    int near_row = i_lo, far_row = i_lo;
    // next row of each kind, clamped to the chunk's last row
    auto next_near = [&]() CSA_INLINE {
        if (near_row + 1 < c1) {
            ++near_row;
            q_row += a.q_ss;
            w_row += a.w_ss;
        }
    };
    auto next_far = [&]() CSA_INLINE {
        if (far_row + 1 < c1) {
            ++far_row;
            s_row += s_stride;
            g_row += a.W;
            seg_row += seg_stride;
        }
    };
    auto fetch_q = [&]() CSA_INLINE {
#pragma unroll
        for (int u = 0; u < G::kPerThread; ++u)
            pre[u] = *reinterpret_cast<const u32x4 *>(q_row + q_off[u]);
        if (w_lane)
            wraw = w_row[tid];
    };
    auto fetch_far = [&](uint32_t (&sp)[G::kSignPerThread], float &gv, int &sv) CSA_INLINE {
#pragma unroll
        for (int u = 0; u < G::kSignPerThread; ++u)
            sp[u] = s_row[s_off[u]];
        gv = g_row[g_off];
        sv = *seg_row;
    };
    auto store = [&](int buf, const uint32_t (&sp)[G::kSignPerThread]) CSA_INLINE {
#pragma unroll
        for (int u = 0; u < G::kPerThread; ++u) {
            const int c = tid + u * kBwdThreads;
            const int h = c / (D / 8), col = (c % (D / 8)) * 8;
            if (c < G::kChunks)
                *reinterpret_cast<u32x4 *>(qbuf(buf) + tile_offset<D>(h, col / 8)) =
                    h < a.H ? pre[u] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < G::kSignPerThread; ++u) {
            const int c = tid + u * kBwdThreads;
            if (c < G::kSignWords)
                sbuf(buf)[c] = (c % NH < a.H && blk0 + c / NH < a.n_blk) ? sp[u] : 0u;
        }
        if (tid < NH)
            wbuf(buf)[tid] = bf16_to_f32(wraw); // heads past H: 0
    };
    // causal threshold of the row after the current one: clamp(floor((off +
    // r + 1) / m), 0, W), carried as quotient and remainder
    int64_t thr_q = floor_div_pos(off + i_lo + 1, a.m);
    int thr_r = (int)(off + i_lo + 1 - thr_q * a.m);
    auto next_thr = [&]() CSA_INLINE {
        const int t = (int)min(max(thr_q, (int64_t)0), (int64_t)a.W);
        if (++thr_r == a.m) {
            thr_r = 0;
            ++thr_q;
        }
        return t;
    };
    // whether (r, j) is unmasked for this lane's entry j
    auto row_ok = [&](int thr, int sv) CSA_INLINE {
        bool ok = j < thr;
        if (a.k_seg)
            ok = ok && kseg == sv;
        return ok;
    };
    // A operand of the dk product for head block hb of the row in buffer
    // buf: lane = entry n, k index r = head 32hb + c_row(r, gi), value
    // g w [l > 0] with the sign of l as the row pass found it
    auto operand = [&](int buf, int hb, float ge, bf16x8 &a0, bf16x8 &a1) CSA_INLINE {
        const float *Wt = wbuf(buf);
        const uint32_t *Sg = sbuf(buf) + wv * NH;
        float pf[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            // c_row(4 q4 + c, gi) = 8 q4 + 4 gi + c: four consecutive heads
            const float4 wq = *reinterpret_cast<const float4 *>(Wt + 32 * hb + 8 * q4 + 4 * gi);
            const uint4 sq = *reinterpret_cast<const uint4 *>(Sg + 32 * hb + 8 * q4 + 4 * gi);
            const float wr[4] = {wq.x, wq.y, wq.z, wq.w};
            const uint32_t sw[4] = {sq.x, sq.y, sq.z, sq.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                // all ones when the logit is positive, else zero
                const int32_t pos = __builtin_amdgcn_sbfe((int32_t)sw[c], sbit, 1);
                // rounded to bf16 by operand_from
                pf[4 * q4 + c] = __int_as_float(pos & __float_as_int(ge * wr[c]));
            }
        }
        a0 = operand_from(pf, 0);
        a1 = operand_from(pf, 8);
    };
    // the q operands of column block c + 1 are read while block c's
    // products run (kept in that order by scheduling barriers)
    auto product = [&](int buf, int hb, const bf16x8 &a0, const bf16x8 &a1) CSA_INLINE {
        const uint16_t *Qh = qbuf(buf) + 32 * hb * D;
        bf16x8 b0 = load_column_operand<D>(Qh, qcol, 0, 0), b1 = load_column_operand<D>(Qh, qcol, 16, 0);
#pragma unroll
        for (int c = 0; c < DB; ++c) {
            bf16x8 n0 = b0, n1 = b1;
            if (c + 1 < DB) {
                n0 = load_column_operand<D>(Qh, qcol, 0, c + 1);
                n1 = load_column_operand<D>(Qh, qcol, 16, c + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            acc[c] = mfma32(a0, b0, acc[c]);
            acc[c] = mfma32(a1, b1, acc[c]);
            __builtin_amdgcn_sched_barrier(0);
            b0 = n0;
            b1 = n1;
        }
    };

    // One row: P = (i - i_lo) % 3 selects the buffers and the slot of row i;
    // (P + 1) % 3 is row i + 1's, (P + 2) % 3 receives row i + 2.  On entry
    // nx0, nx1 hold row i's first head-block operand and thr_i its threshold;
    // on exit they hold row i + 1's.  Rows past the chunk are loaded,
    // stored and given operands, never multiplied.
    bf16x8 nx0, nx1;
    int thr_i;
    auto row_step = [&](int i, auto P_) CSA_INLINE {
        constexpr int P = decltype(P_)::value, P1 = (P + 1) % 3, P2 = (P + 2) % 3;
        const bool ok = row_ok(thr_i, ssl[P]);
        const float ge = ok ? gsl[P] : 0.0f;
        const int thr_n = next_thr();
        const float ge_n = row_ok(thr_n, ssl[P1]) ? gsl[P1] : 0.0f;
        next_near();
        fetch_q(); // row i + 2
        next_far();
        fetch_far(sgn[P], gsl[P], ssl[P]); // row i + 3
        // the loads go out first, the next row's operand is built before
        // the barrier (scheduling barriers keep both where they are)
        __builtin_amdgcn_sched_barrier(0);
        if (wave_has && ballot(ok) != 0) {
            product(P, 0, nx0, nx1);
            // rolled: fewer live registers
#pragma unroll 1
            for (int hb = 1; hb < HB; ++hb) {
                bf16x8 a0, a1;
                operand(P, hb, ge, a0, a1);
                product(P, hb, a0, a1);
            }
        }
        operand(P1, 0, ge_n, nx0, nx1);
        // consumed here, so the compiler cannot sink the work past the barrier
        __asm__ volatile("" ::"v"(nx0), "v"(nx1));
        __builtin_amdgcn_sched_barrier(0);
        thr_i = thr_n;
        store(P2, sgn[P2]); // row i + 2 (after the chunk's last row: stored, never read)
        __syncthreads();
    };

    // Two deep (four head blocks): row i's buffer and slot P = (i - i_lo) % 2;
    // the q block of row i + 1 is loaded and stored during row i, its far
    // values two rows ahead, and each head block's operand is built in turn.
    auto row_step2 = [&](int i, auto P_) CSA_INLINE {
        constexpr int P = decltype(P_)::value, P1 = P ^ 1;
        const bool ok = row_ok(thr_i, ssl[P]);
        const float ge = ok ? gsl[P] : 0.0f;
        thr_i = next_thr();
        next_near();
        fetch_q(); // row i + 1
        next_far();
        fetch_far(sgn[P], gsl[P], ssl[P]); // row i + 2
        if (wave_has && ballot(ok) != 0) {
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                bf16x8 a0, a1;
                operand(P, hb, ge, a0, a1);
                product(P, hb, a0, a1);
            }
        }
        store(P1, sgn[P1]); // row i + 1 (after the chunk's last row: stored, never read)
        __syncthreads();
    };
    if constexpr (G::kDeep == 2) {
        fetch_q();
        fetch_far(sgn[0], gsl[0], ssl[0]);
        next_far();
        fetch_far(sgn[1], gsl[1], ssl[1]);
        store(0, sgn[0]);
        // Every load issued so far completes here (see the row pass).
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        thr_i = next_thr();
        for (int i = i_lo; i < c1; i += 2) {
            row_step2(i, std::integral_constant<int, 0>());
            if (i + 1 < c1)
                row_step2(i + 1, std::integral_constant<int, 1>());
        }
    } else {
    // prologue: rows i_lo and i_lo + 1 stored, far rows i_lo .. i_lo + 2
    // loaded, row i_lo's first operand built
    fetch_q();
    fetch_far(sgn[0], gsl[0], ssl[0]);
    next_far();
    fetch_far(sgn[1], gsl[1], ssl[1]);
    next_far();
    fetch_far(sgn[2], gsl[2], ssl[2]);
    store(0, sgn[0]);
    next_near();
    fetch_q();
    // Every load issued so far completes here (see the row pass).
    __builtin_amdgcn_s_waitcnt(0);
    store(1, sgn[1]);
    __syncthreads();
    thr_i = next_thr();
    operand(0, 0, row_ok(thr_i, ssl[0]) ? gsl[0] : 0.0f, nx0, nx1);
    for (int i = i_lo; i < c1; i += 3) {
        row_step(i, std::integral_constant<int, 0>());
        if (i + 1 < c1)
            row_step(i + 1, std::integral_constant<int, 1>());
        if (i + 2 < c1)
            row_step(i + 2, std::integral_constant<int, 2>());
    }
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
    // the partials of kBatch chunks are read together (one memory latency
    // per batch, not per chunk) and added in chunk order
    constexpr int kBatch = 8;
    const int64_t off = row_offset(a, b); // (chunk_live, with the offset read once)
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int c0 = 0; c0 < a.n_chunks; c0 += kBatch) {
        float4 p[kBatch];
        bool live[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int c = c0 + u;
            const int last = min((c + 1) * kBwdChunkRows, a.S) - 1;
            live[u] = c < a.n_chunks && visible_entries(off + last, a.m, a.W) > jtile0;
            p[u] = live[u] ? *reinterpret_cast<const float4 *>(a.part + (((int64_t)b * a.n_chunks + c) * a.W) * D + e)
                           : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (live[u]) {
                s.x += p[u].x;
                s.y += p[u].y;
                s.z += p[u].z;
                s.w += p[u].w;
            }
        }
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
