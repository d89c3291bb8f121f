// The indexer score of one query row against a tile of 64 compressed
// entries, on MFMA.
//
// For query row i the heads are the MFMA M dimension and the entries the N
// dimension: D(32 heads x 32 entries) = Q_i(32 heads x 16 of D) * K^T(16 of D x
// 32 entries), accumulated over D in fp32 (v_mfma_f32_32x32x16_bf16, the
// full-rate bf16 MFMA on gfx950).  Each lane then holds 16 heads of one entry,
// so the ReLU and the head-weighted sum run in registers (integer max + fma
// per head), and one cross-half lane swap per 64 entries finishes the sum over
// heads.  The per-head logits never leave the register file.
//
// Every kernel computes scores through tile_scores(), so every plan yields
// the same fp32 bits.
#pragma once

#include "csa_device.hpp"

namespace csa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.  Lane l
// supplies A row (l % 32), B column (l % 32) and eight consecutive k values
// selected by l / 32; it receives D column (l % 32), rows
// 8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.  A and B use the same k
// assignment, so any consistent placement of the contraction index inside a
// fragment yields the same dot products.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Head of accumulator register r in lane group g (= lane / 32) of a 32-head block.
__host__ __device__ constexpr int c_row(int r, int g) { return 8 * (r / 4) + 4 * g + (r % 4); }

// ReLU on fp32 through the integer max: every negative float (and -0) has a
// negative int32 image, so max(bits, 0) is +0 for them and the identity for
// positive values.  One VALU op, exact.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// One query row resident in registers: A fragments of every 32-head block and
// 16-wide k-step, plus this lane's head weights (heads 32*hb + c_row(r, lane/32)).
template <int HB, int KS>
struct RowOperand {
    bf16x8 a[HB][KS];
    float w[HB][16];
};

// q_row = q + b*q_sb + i*q_ss, w_row = w + b*w_sb + i*w_ss.  Heads >= H get
// weight zero and the (finite) queries of head H-1, so they add exact zeros.
// Loads are issued unconditionally so they can all be in flight at once.
// With full head blocks (H == 32*HB) and an 8-byte aligned weight row, a
// lane's loads are one base address per head block with immediate offsets:
// its 8-byte runs of 4 consecutive weights (heads 32hb + 8j + 4g .. +3) and
// its 16-byte query fragments; nothing consumes them before the first
// tile, so they stay in flight while the workgroup stages its first key tile.
template <int HB, int KS>
__device__ __forceinline__ void load_row(RowOperand<HB, KS> &r, const uint16_t *q_row, int64_t q_sh,
                                         const uint16_t *w_row, int H)
{
    // lane-derived addresses stay local to the call (see opaque_lane)
    const int l = opaque_lane();
    const int n = l & 31, g = l >> 5;
    if (H == 32 * HB && (reinterpret_cast<uintptr_t>(w_row) & 7u) == 0) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const uint16_t *p = q_row + (int64_t)(hb * 32 + n) * q_sh + 8 * g;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                r.a[hb][s] = load_frag(p + 16 * s);
        }
        uint2 wv[HB][4];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wv[hb][j] = *reinterpret_cast<const uint2 *>(w_row + hb * 32 + 8 * j + 4 * g);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // c_row(4j + c, g) = 8j + 4g + c
                r.w[hb][4 * j + 0] = __uint_as_float(wv[hb][j].x << 16);
                r.w[hb][4 * j + 1] = __uint_as_float(wv[hb][j].x & 0xFFFF0000u);
                r.w[hb][4 * j + 2] = __uint_as_float(wv[hb][j].y << 16);
                r.w[hb][4 * j + 3] = __uint_as_float(wv[hb][j].y & 0xFFFF0000u);
            }
        return;
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int h = hb * 32 + n;
        const uint16_t *p = q_row + (int64_t)min(h, H - 1) * q_sh + 8 * g;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            r.a[hb][s] = load_frag(p + 16 * s);
    }
    uint16_t wb[HB][16];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            wb[hb][rr] = w_row[min(hb * 32 + c_row(rr, g), H - 1)];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            r.w[hb][rr] = (hb * 32 + c_row(rr, g) < H) ? bf16_to_f32(wb[hb][rr]) : 0.0f;
}

// B fragments of 32 entries staged in LDS with a row pitch of `pitch`
// elements: lane l reads entry (l % 32), 8 values at 16*s + 8*(l/32).
template <int KS>
__device__ __forceinline__ void load_entries_lds(bf16x8 (&b)[KS], const uint16_t *tile, int entry0, int pitch)
{
    const int l = lane();
    const uint16_t *p = tile + (entry0 + (l & 31)) * pitch + 8 * (l >> 5);
#pragma unroll
    for (int s = 0; s < KS; ++s)
        b[s] = load_frag(p + 16 * s);
}

// B fragments straight from global memory.  Entries at or beyond `limit`
// (always masked by the caller) are not read: those lanes read entry
// entry0 instead, which is below the limit.
template <int KS>
__device__ __forceinline__ void load_entries_global(bf16x8 (&b)[KS], const uint16_t *k_batch, int64_t k_sw,
                                                    int entry0, int limit)
{
    const int l = lane();
    int j = entry0 + (l & 31);
    j = j < limit ? j : entry0;
    const uint16_t *p = k_batch + (int64_t)j * k_sw + 8 * (l >> 5);
#pragma unroll
    for (int s = 0; s < KS; ++s)
        b[s] = load_frag(p + 16 * s);
}

// Per-head logits of 32 entries: c[hb] = Q(heads 32hb..32hb+31) . K^T.
template <int HB, int KS>
__device__ __forceinline__ void subtile_logits(f32x16 (&c)[HB], const RowOperand<HB, KS> &r, const bf16x8 (&b)[KS])
{
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
        c[hb] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
            c[hb] = mfma32(r.a[hb][s], b[s], c[hb]);
}

// This lane's share of the unscaled score of entry (lane % 32): the sum over
// its 16 heads of every 32-head block, w_h * ReLU(logit_h).  Each head block
// has its own fma chain; the chains are added in a fixed order.
template <int HB, int KS>
__device__ __forceinline__ float logits_partial(const RowOperand<HB, KS> &r, const f32x16 (&c)[HB])
{
    float acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        acc[hb] = 0.0f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            acc[hb] = __builtin_fmaf(r.w[hb][rr], relu(c[hb][rr]), acc[hb]);
    }
#pragma unroll
    for (int step = 1; step < HB; step <<= 1)
#pragma unroll
        for (int hb = 0; hb + step < HB; hb += 2 * step)
            acc[hb] += acc[hb + step];
    return acc[0];
}

template <int HB, int KS>
__device__ __forceinline__ float subtile_partial(const RowOperand<HB, KS> &r, const bf16x8 (&b)[KS])
{
    f32x16 c[HB];
    subtile_logits<HB, KS>(c, r, b);
    return logits_partial<HB, KS>(r, c);
}

// Combine the lane shares of two 32-entry subtiles (entries j0..j0+31 in p0,
// j0+32..j0+63 in p1): after one swap of lane halves, lane l holds the full
// unscaled score of entry j0 + l (its own half's share plus the other half's,
// low half first).
__device__ __forceinline__ float combine_halves(float p0, float p1)
{
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Apply the scale once and turn a -0 result into +0.
__device__ __forceinline__ float scaled_score(float acc, float scale) { return acc * scale + 0.0f; }

} // namespace csa
