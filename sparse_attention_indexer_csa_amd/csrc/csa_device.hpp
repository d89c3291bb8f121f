// Device primitives for the gfx950 indexer kernels: bf16 MFMA fragments,
// orderable score keys and wave-level helpers.  Wavefronts are 64 lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane() { return (int)__lane_id(); }

// 16 bytes from memory reinterpreted as eight bf16 values.
__device__ __forceinline__ bf16x8 load_frag(const uint16_t *p)
{
    u32x4 v = *reinterpret_cast<const u32x4 *>(p);
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 zero_frag()
{
    u32x4 v = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l % 16), B column (l % 16), eight consecutive k
// values selected by l / 16, and receives D column (l % 16), rows
// 4*(l/16) .. 4*(l/16)+3.  A and B use the same k assignment, so any
// consistent placement of the contraction index inside a fragment yields the
// same dot products.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Monotone map of fp32 scores onto uint32: a larger score gives a larger key,
// -0 and +0 give the same key.  -inf maps to 0x007FFFFF and NaNs fall outside
// (0x007FFFFF, 0xFF800000], which is exactly the set of selectable keys.
__device__ __forceinline__ uint32_t score_key(float s)
{
    // -0 becomes +0 (on the bits, so no float mode can touch denormals);
    // negative floats then flip all bits, non-negative ones only the sign
    uint32_t u = __float_as_uint(s);
    u = (u == 0x80000000u) ? 0u : u;
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

constexpr uint32_t kKeyNegInf = 0x007FFFFFu;
constexpr uint32_t kKeyPosInf = 0xFF800000u;

__device__ __forceinline__ bool key_selectable(uint32_t key) { return key > kKeyNegInf && key <= kKeyPosInf; }

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int rank_below(uint64_t mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// The lane index as a value the compiler cannot hoist out of an enclosing
// loop: code that derives many lane masks from it (sorting networks) keeps
// them local instead of holding them in registers across the loop.
__device__ __forceinline__ int opaque_lane()
{
    int l = lane();
    __asm__ volatile("" : "+v"(l));
    return l;
}

// v in an SGPR of its own.  A scalar read from the argument block otherwise
// shares its register tuple with its neighbours; when register pressure
// spills the tuple, every use restores all of it.
__device__ __forceinline__ int own_sgpr(int v)
{
    __asm__ volatile("" : "+s"(v));
    return v;
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uniform_u(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

__device__ __forceinline__ int read_lane(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

// Exclusive prefix sum over the 64 lanes of a wave.
// Inclusive prefix sum over the 64 lanes with DPP: shifts of 1, 2, 4, 8
// inside each 16-lane row, then the last lane of row r is added to the rows
// above it (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3).
__device__ __forceinline__ int wave_inclusive_sum(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false); // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false); // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false); // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false); // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false); // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false); // row_bcast:31
    return x;
}

__device__ __forceinline__ int wave_exclusive_sum(int v) { return wave_inclusive_sum(v) - v; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask)
{
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = (uint32_t)__shfl_xor((int)lo, mask, kWave);
    hi = (uint32_t)__shfl_xor((int)hi, mask, kWave);
    return ((uint64_t)hi << 32) | lo;
}

// Orders the LDS traffic of one wave: everything issued before is complete
// and visible to the wave's lanes before anything issued after.
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Floor division for a positive divisor.
__device__ __forceinline__ int64_t floor_div_pos(int64_t a, int64_t m)
{
    int64_t q = a / m;
    return (a % m != 0 && a < 0) ? q - 1 : q;
}

// Visible compressed entries for a row at absolute position pos.
__device__ __forceinline__ int visible_entries(int64_t pos, int m, int W)
{
    int64_t t = floor_div_pos(pos + 1, m);
    t = t < 0 ? 0 : t;
    t = t > W ? W : t;
    return (int)t;
}

} // namespace csa
