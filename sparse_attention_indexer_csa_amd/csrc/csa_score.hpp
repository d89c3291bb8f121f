// The indexer score of one query row against 16 compressed entries, on MFMA.
//
// For query row i the heads are the MFMA M dimension and the entries the N
// dimension: D(16 heads x 16 entries) = Q_i(16 heads x 32 of D) * K^T(32 of D x
// 16 entries), accumulated over D in fp32.  Each lane then holds 4 heads of
// one entry, so the ReLU and the head-weighted sum run in registers
// (max + fma per head), and two cross-lane adds finish the sum over heads.
// The per-head logits never leave the register file.
//
// Every kernel calls subtile_score(), so every plan yields the same fp32 bits.
#pragma once

#include "csa_device.hpp"

namespace csa {

// One query row resident in registers: A fragments of every 16-head block and
// k-step, plus this lane's head weights (heads 16*hb + 4*(lane/16) + r).
template <int HB, int KS>
struct RowOperand {
    bf16x8 a[HB][KS];
    float w[HB][4];
};

// q_row = q + b*q_sb + i*q_ss, w_row = w + b*w_sb + i*w_ss.  Heads >= H read
// as zero queries with zero weight, which adds exact zeros.
template <int HB, int KS>
__device__ __forceinline__ void load_row(RowOperand<HB, KS> &r, const uint16_t *q_row, int64_t q_sh,
                                         const uint16_t *w_row, int H)
{
    const int l = lane();
    const int n = l & 15, g = l >> 4;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int h = hb * 16 + n;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            r.a[hb][s] = (h < H) ? load_frag(q_row + (int64_t)h * q_sh + s * 32 + 8 * g) : zero_frag();
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int h = hb * 16 + 4 * g + rr;
            r.w[hb][rr] = (h < H) ? bf16_to_f32(w_row[h]) : 0.0f;
        }
}

// B fragments of 16 entries staged in LDS with a row pitch of `pitch`
// elements: lane l reads entry (l % 16), 8 values at 32*s + 8*(l/16).
template <int KS>
__device__ __forceinline__ void load_entries_lds(bf16x8 (&b)[KS], const uint16_t *tile, int entry0, int pitch)
{
    const int l = lane();
    const uint16_t *p = tile + (entry0 + (l & 15)) * pitch + 8 * (l >> 4);
#pragma unroll
    for (int s = 0; s < KS; ++s)
        b[s] = load_frag(p + 32 * s);
}

// B fragments straight from global memory; entries at or beyond `limit`
// are not read (zero fragments).
template <int KS>
__device__ __forceinline__ void load_entries_global(bf16x8 (&b)[KS], const uint16_t *k_batch, int64_t k_sw,
                                                    int entry0, int limit)
{
    const int l = lane();
    const int j = entry0 + (l & 15);
    const uint16_t *p = k_batch + (int64_t)j * k_sw + 8 * (l >> 4);
#pragma unroll
    for (int s = 0; s < KS; ++s)
        b[s] = (j < limit) ? load_frag(p + 32 * s) : zero_frag();
}

// Unscaled score sum_h w_h * ReLU(q_h . k_j) of entry (lane % 16); the four
// lane groups return the same bits.
template <int HB, int KS>
__device__ __forceinline__ float subtile_score(const RowOperand<HB, KS> &r, const bf16x8 (&b)[KS])
{
    f32x4 c[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
        c[hb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
            c[hb] = mfma16(r.a[hb][s], b[s], c[hb]);
    float acc = 0.0f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            acc = __builtin_fmaf(r.w[hb][rr], fmaxf(c[hb][rr], 0.0f), acc);
    acc += __shfl_xor(acc, 16, kWave);
    acc += __shfl_xor(acc, 32, kWave);
    return acc;
}

// Apply the scale once and turn a -0 result into +0.
__device__ __forceinline__ float scaled_score(float acc, float scale) { return acc * scale + 0.0f; }

} // namespace csa
