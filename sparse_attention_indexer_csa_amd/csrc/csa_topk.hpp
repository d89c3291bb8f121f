// Exact per-row top-k.
//
// Wave level (TopKRow): one wave owns a row and receives its (key, entry)
// pairs 64 at a time in increasing entry order.  It keeps a candidate buffer
// of `cap` pairs in LDS and a threshold tau: a pair may enter only if its key
// is > tau.  When the buffer would overflow, one histogram over the buffer's
// key range finds the bucket of the k-th largest key, an order-preserving
// compaction keeps every key at or above that bucket (at least k pairs), and
// tau becomes the bucket's lower bound minus one; if that would free too
// little room, a radix select finds T, the k-th largest key in the buffer,
// and the compaction keeps every key > T plus the earliest keys == T, k pairs
// in all, with tau = T.  A later pair with key <= tau can never make the top
// k: k kept pairs beat it (larger key, or equal key and lower entry).  At the
// end a final select (the radix select, or its version over registers in the
// row kernels) leaves exactly min(k, count) pairs, which a bitonic sort
// orders by (key descending, entry ascending).
//
// Block level (block_select_sort): several waves that each hold a candidate
// buffer for a contiguous segment of one row (segments in increasing entry
// order) run one shared radix select over the union, keep the winners in
// entry order, and one wave sorts them.
//
// Keys are score_key() images of fp32 scores, so key order is score order and
// -0 ties with +0.
#pragma once

#include "csa_device.hpp"
#include "csa_launch.hpp"

namespace csa {

template <typename EntT>
struct TopKRow {
    uint32_t *key;  // LDS [cap]
    EntT *ent;      // LDS [cap]
    uint32_t *hist; // LDS [256], scratch of the owning wave
    int cap;        // >= k + 64
    int k;
    int count;      // wave-uniform
    uint32_t tau;   // wave-uniform, never below kKeyNegInf (the key of -inf)
};

template <typename EntT>
__device__ __forceinline__ void topk_init(TopKRow<EntT> &t, uint32_t *key, EntT *ent, uint32_t *hist, int cap, int k)
{
    t.key = key;
    t.ent = ent;
    t.hist = hist;
    t.cap = cap;
    t.k = k;
    t.count = 0;
    t.tau = kKeyNegInf;
}

// Digit search shared by the wave and block selects: hist holds 256 counts
// of the current digit; find the digit d such that fewer than kk keys lie in
// higher digits and at least kk in digits >= d.  Returns d; `above` receives
// the count in higher digits.  Run by one whole wave.
__device__ __forceinline__ int find_digit(const uint32_t *hist, int kk, int &above)
{
    const int l = lane();
    // lane l owns digits 255-4l, 254-4l, 253-4l, 252-4l (descending)
    int h[4], tot = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        h[r] = (int)hist[255 - 4 * l - r];
        tot += h[r];
    }
    int cum = wave_exclusive_sum(tot);
    int found = -1, ab = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (found < 0 && cum < kk && kk <= cum + h[r]) {
            found = 255 - 4 * l - r;
            ab = cum;
        }
        cum += h[r];
    }
    const uint64_t bal = ballot(found >= 0);
    const int src = bal ? (int)__builtin_ctzll(bal) : 0;
    above = read_lane(ab, src);
    return read_lane(found, src) & 0xFF;
}

// Value of v in lane (lane ^ LX), with VALU lane exchanges only: DPP quad
// permutations for distances 1 and 2, a half-row mirror followed by a quad
// reversal for 4, a row rotation for 8, and the gfx950 lane-swap
// instructions for 16 and 32 (v passed as both operands; each lane keeps the
// half that came from the other row / half).
template <int LX>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v)
{
    if constexpr (LX == 1)
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false); // quad_perm [1,0,3,2]
    else if constexpr (LX == 2)
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false); // quad_perm [2,3,0,1]
    else if constexpr (LX == 4) {
        const int m = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false); // row_half_mirror
        return (uint32_t)__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false);    // quad_perm [3,2,1,0]
    } else if constexpr (LX == 8)
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false); // row_ror:8
    else if constexpr (LX == 16) {
        const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return ((lane() >> 4) & 1) ? sw[0] : sw[1];
    } else {
        static_assert(LX == 32, "lane distance must be a power of two below 64");
        const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane() < 32) ? sw[1] : sw[0];
    }
}

// The lanes whose index has bit b clear (b a power of two; 64: every lane).
__device__ __forceinline__ constexpr uint64_t lanes_bit_clear(int b)
{
    return b == 1 ? 0x5555555555555555ull : b == 2 ? 0x3333333333333333ull
         : b == 4 ? 0x0F0F0F0F0F0F0F0Full : b == 8 ? 0x00FF00FF00FF00FFull
         : b == 16 ? 0x0000FFFF0000FFFFull : b == 32 ? 0x00000000FFFFFFFFull : ~0ull;
}

// Whether to take x for max(x, y) on the lanes of `hi` and min(x, y) on the
// others: one compare, a scalar operation on the lane masks, no per-lane
// direction arithmetic.
__device__ __forceinline__ bool take_first(uint64_t hi, uint64_t x, uint64_t y)
{
    return (x > y) == __builtin_amdgcn_inverse_ballot_w64(hi);
}

// All ones in the lanes of m, a lane mask known at compile time, zero in
// the others.  The mask passes through an empty asm, so the select is made
// where it is used instead of being hoisted out of enclosing loops.
__device__ __forceinline__ uint32_t lane_sel(uint64_t m)
{
    __asm__ volatile("" : "+s"(m));
    return __builtin_amdgcn_inverse_ballot_w64(m) ? 0xFFFFFFFFu : 0u;
}

// The buffer passes below read the keys in batches of kPassBatch chunks of 64
// (the reads of a batch are in flight together, indexes past the end clamped
// to the last key) instead of one dependent read per chunk.
constexpr int kPassBatch = 4;

// Smallest and largest key of key[0..count), count >= 1.  (A clamped
// duplicate of the last key changes neither.)
__device__ __forceinline__ void key_range(const uint32_t *key, int count, uint32_t &lo, uint32_t &hi)
{
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    const int l = lane();
#pragma unroll 1
    for (int b0 = 0; b0 < count; b0 += kPassBatch * kWave) {
        uint32_t kv[kPassBatch];
#pragma unroll
        for (int c = 0; c < kPassBatch; ++c)
            kv[c] = key[min(b0 + c * kWave + l, count - 1)];
#pragma unroll
        for (int c = 0; c < kPassBatch; ++c) {
            mn = min(mn, kv[c]);
            mx = max(mx, kv[c]);
        }
    }
    mn = min(mn, lane_xor_u32<1>(mn));
    mx = max(mx, lane_xor_u32<1>(mx));
    mn = min(mn, lane_xor_u32<2>(mn));
    mx = max(mx, lane_xor_u32<2>(mx));
    mn = min(mn, lane_xor_u32<4>(mn));
    mx = max(mx, lane_xor_u32<4>(mx));
    mn = min(mn, lane_xor_u32<8>(mn));
    mx = max(mx, lane_xor_u32<8>(mx));
    mn = min(mn, lane_xor_u32<16>(mn));
    mx = max(mx, lane_xor_u32<16>(mx));
    mn = min(mn, lane_xor_u32<32>(mn));
    mx = max(mx, lane_xor_u32<32>(mx));
    lo = uniform_u(mn);
    hi = uniform_u(mx);
}

// Histogram of the keys in [base, base + span] by (key - base) >> shift
// (at most 256 buckets), then the bucket holding the kk-th largest of them.
__device__ __forceinline__ int bucket_of_kth(const uint32_t *key, int count, uint32_t base, uint32_t span, int shift,
                                             int kk, uint32_t *hist, int &above)
{
    for (int b = lane(); b < 256; b += kWave)
        hist[b] = 0u;
    wave_lds_fence();
    const int l = lane();
#pragma unroll 1
    for (int b0 = 0; b0 < count; b0 += kPassBatch * kWave) {
        uint32_t kv[kPassBatch];
#pragma unroll
        for (int c = 0; c < kPassBatch; ++c)
            kv[c] = key[min(b0 + c * kWave + l, count - 1)];
#pragma unroll
        for (int c = 0; c < kPassBatch; ++c) {
            const uint32_t off = kv[c] - base;
            if (b0 + c * kWave + l < count && off <= span)
                atomicAdd(&hist[off >> shift], 1u);
        }
    }
    wave_lds_fence();
    const int d = find_digit(hist, kk, above);
    wave_lds_fence();
    return d;
}

// Bitonic sort of one u32 per lane (64 values) into descending lane order.
template <int SIZE, int STRIDE>
__device__ __forceinline__ uint32_t bitonic_u32_level(uint32_t v, int l)
{
    const uint32_t o = lane_xor_u32<STRIDE>(v);
    const bool keep_max = ((l & STRIDE) == 0) == ((l & SIZE) == 0);
    v = keep_max ? max(v, o) : min(v, o);
    if constexpr (STRIDE > 1)
        return bitonic_u32_level<SIZE, STRIDE / 2>(v, l);
    else
        return v;
}

template <int SIZE = 2>
__device__ __forceinline__ uint32_t sort_u32_desc(uint32_t v, int l)
{
    v = bitonic_u32_level<SIZE, SIZE / 2>(v, l);
    if constexpr (SIZE < kWave)
        return sort_u32_desc<SIZE * 2>(v, l);
    else
        return v;
}

// The n (<= 64) keys of key[0..count) that lie in [base, base + span], one
// per lane (lane order = buffer order; lanes >= n get 0, below every
// selectable key).  `scratch` holds at least 64 words.
__device__ __forceinline__ uint32_t gather_range(const uint32_t *key, int count, uint32_t base, uint32_t span, int n,
                                                 uint32_t *scratch)
{
    int out = 0;
#pragma unroll 1
    for (int b0 = 0; b0 < count && out < n; b0 += kWave) {
        const int i = b0 + lane();
        const uint32_t kv = i < count ? key[i] : 0u;
        const bool in = i < count && kv - base <= span;
        const uint64_t bal = ballot(in);
        if (in)
            scratch[out + rank_below(bal)] = kv;
        out += popc64(bal);
    }
    wave_lds_fence();
    const uint32_t x = lane() < n ? scratch[lane()] : 0u;
    wave_lds_fence();
    return x;
}

// Radix select over key[0..count), count > k: the k-th largest key T, and how
// many keys equal to T belong to the top k (the earliest ones in buffer order).
// The digits adapt to the keys' actual range: each pass splits the current
// range [base, base + span] into at most 256 buckets, so scores that share
// their leading bits still spread over many buckets.  Once the bucket that
// holds the k-th key has at most 64 keys, they are gathered into one
// register per lane and sorted there instead of running more passes.
__device__ __forceinline__ void radix_select(const uint32_t *key, int count, int k, uint32_t *hist, uint32_t &T,
                                             int &ties_keep)
{
    wave_lds_fence();
    uint32_t base, hi;
    key_range(key, count, base, hi);
    uint32_t span = hi - base;
    int kk = k;
#pragma unroll 1
    while (span != 0u) {
        const int bits = 32 - __builtin_clz(span);
        const int shift = bits > 8 ? bits - 8 : 0;
        int above;
        const uint32_t d = (uint32_t)bucket_of_kth(key, count, base, span, shift, kk, hist, above);
        const int inb = uniform((int)hist[d]);
        kk -= above;
        base += d << shift;
        if (shift == 0)
            break;
        span = min(span - (d << shift), (1u << shift) - 1u);
        if (inb <= kWave) {
            wave_lds_fence();
            const uint32_t sx = sort_u32_desc(gather_range(key, count, base, span, inb, hist), lane());
            T = uniform_u(read_lane((int)sx, kk - 1));
            ties_keep = kk - popc64(ballot(sx > T));
            return;
        }
    }
    T = base;
    ties_keep = kk;
}

// Keep keys > T and the first ties_keep keys == T, in place and in order.
// Returns the new count.  A batch is read before any of it is written: the
// kept pairs of a chunk land at or below the chunk's own positions, so no
// write reaches a pair not yet read.
template <typename EntT>
__device__ __forceinline__ int compact_keep(uint32_t *key, EntT *ent, int count, uint32_t T, int ties_keep)
{
    int out = 0, ties = 0;
    const int l = lane();
#pragma unroll 1
    for (int b0 = 0; b0 < count; b0 += kPassBatch * kWave) {
        uint32_t kv[kPassBatch];
        EntT ev[kPassBatch];
#pragma unroll
        for (int c = 0; c < kPassBatch; ++c) {
            const int i = min(b0 + c * kWave + l, count - 1);
            kv[c] = key[i];
            ev[c] = ent[i];
        }
#pragma unroll
        for (int c = 0; c < kPassBatch; ++c) {
            const bool in = b0 + c * kWave + l < count;
            const bool eq = in && kv[c] == T;
            const uint64_t beq = ballot(eq);
            const bool keep = (in && kv[c] > T) || (eq && ties + rank_below(beq) < ties_keep);
            ties += popc64(beq);
            const uint64_t bk = ballot(keep);
            if (keep) {
                const int pos = out + rank_below(bk);
                key[pos] = kv[c];
                ent[pos] = ev[c];
            }
            out += popc64(bk);
        }
    }
    wave_lds_fence();
    return out;
}

// Reduce the buffer to exactly its top k (no-op when it holds at most k pairs).
template <typename EntT>
__device__ __forceinline__ void topk_reduce(TopKRow<EntT> &t)
{
    if (t.count > t.k) {
        uint32_t T;
        int keep;
        radix_select(t.key, t.count, t.k, t.hist, T, keep);
        t.count = uniform(compact_keep(t.key, t.ent, t.count, T, keep));
        t.tau = uniform_u(T);
    }
}

// Make room in a full buffer cheaply: one range-adaptive histogram finds the
// bucket holding the k-th largest key; every key at or above that bucket's
// lower bound L is kept (at least k of them) and tau becomes L - 1.  A later
// pair with key < L is beaten by those k kept keys, so dropping it is exact.
// Falls back to the exact reduction when that would free too little.
template <typename EntT>
__device__ __forceinline__ void topk_make_room(TopKRow<EntT> &t)
{
    wave_lds_fence();
    uint32_t lo, hi;
    key_range(t.key, t.count, lo, hi);
    const uint32_t span = hi - lo;
    if (span != 0u) {
        const int bits = 32 - __builtin_clz(span);
        const int shift = bits > 8 ? bits - 8 : 0;
        int above;
        const uint32_t d = (uint32_t)bucket_of_kth(t.key, t.count, lo, span, shift, t.k, t.hist, above);
        const int kept = above + (int)t.hist[d];
        if (d > 0u && kept + 2 * kWave <= t.cap) {
            const uint32_t L = lo + (d << shift);
            t.count = uniform(compact_keep(t.key, t.ent, t.count, L - 1u, 0));
            t.tau = uniform_u(L - 1u);
            return;
        }
    }
    topk_reduce(t);
}

// Offer one pair per lane; lanes must hold increasing entries, and every pair
// offered later must have a larger entry.
template <typename EntT>
__device__ __forceinline__ void topk_push(TopKRow<EntT> &t, uint32_t kv, uint32_t entry, bool valid)
{
    bool pass = valid && kv > t.tau;
    uint64_t bal = ballot(pass);
    int n = popc64(bal);
    if (t.count + n > t.cap) {
        topk_make_room(t);
        pass = valid && kv > t.tau;
        bal = ballot(pass);
        n = popc64(bal);
    }
    if (pass) {
        const int pos = t.count + rank_below(bal);
        t.key[pos] = kv;
        t.ent[pos] = (EntT)entry;
    }
    t.count += n;
}

// The push without a capacity check, for code that keeps count + 64 <= cap
// itself (topk_reserve).
template <typename EntT>
__device__ __forceinline__ void topk_push_unchecked(TopKRow<EntT> &t, uint32_t kv, uint32_t entry, bool valid)
{
    const bool pass = valid && kv > t.tau;
    const uint64_t bal = ballot(pass);
    if (pass) {
        const int pos = t.count + rank_below(bal);
        t.key[pos] = kv;
        t.ent[pos] = (EntT)entry;
    }
    t.count += popc64(bal);
}

// Room for one more push of 64 pairs.
template <typename EntT>
__device__ __forceinline__ void topk_reserve(TopKRow<EntT> &t)
{
    if (t.count + kWave > t.cap)
        topk_make_room(t);
}

// ---------------------------------------------------------------------------
// Bitonic sort of 64*E values held by one wave, lane l holding elements
// l*E .. l*E+E-1, into descending order.  Partners in other lanes come from
// lane_xor_u32 (VALU exchanges only); partners inside a lane are plain
// registers.
// ---------------------------------------------------------------------------
// One cross-lane stage: partners at lane distance LX.  For these stages the
// keep-larger flag depends only on the lane (stride and size are multiples
// of E), so it is computed once.
template <int LX, int E>
__device__ __forceinline__ void cross_stage(uint64_t (&v)[E], bool keep_max)
{
    uint32_t ohi[E], olo[E];
#pragma unroll
    for (int r = 0; r < E; ++r) {
        ohi[r] = lane_xor_u32<LX>((uint32_t)(v[r] >> 32));
        olo[r] = lane_xor_u32<LX>((uint32_t)v[r]);
    }
    // distinct composites: keep v when (v > o) matches keep_max
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const uint64_t o = ((uint64_t)ohi[r] << 32) | olo[r];
        v[r] = ((v[r] < o) != keep_max) ? v[r] : o;
    }
}

template <int E>
__device__ __forceinline__ void bitonic_in_lane(uint64_t (&v)[E], int size, int l)
{
#pragma unroll
    for (int stride = E / 2; stride >= 1; stride >>= 1) {
        if (stride < size) {
#pragma unroll
            for (int r = 0; r < E; ++r) {
                if ((r & stride) == 0) {
                    const bool desc = ((l * E + r) & size) == 0;
                    const uint64_t a = v[r], b = v[r + stride];
                    const bool sw = desc ? (a < b) : (a > b);
                    v[r] = sw ? b : a;
                    v[r + stride] = sw ? a : b;
                }
            }
        }
    }
}

// In-lane stages of one level with the block size known at compile time.
// Element r of lane l sorts descending iff bit SIZE of l*E + r is clear:
// for SIZE < E that is a constant of r, otherwise it depends on the lane
// only.  The composites are distinct, so "a > b" is "not a < b".
template <int E, int SIZE>
__device__ __forceinline__ void bitonic_in_lane_fixed(uint64_t (&v)[E], int l)
{
    const bool asc_lane = ((l * E) & SIZE) != 0;
#pragma unroll
    for (int stride = (SIZE / 2 < E / 2 ? SIZE / 2 : E / 2); stride >= 1; stride >>= 1) {
#pragma unroll
        for (int r = 0; r < E; ++r) {
            if ((r & stride) == 0) {
                const uint64_t a = v[r], b = v[r + stride];
                const bool lt = a < b;
                bool sw;
                if constexpr (SIZE >= E)
                    sw = lt != asc_lane;
                else
                    sw = ((r & SIZE) == 0) ? lt : !lt;
                v[r] = sw ? b : a;
                v[r + stride] = sw ? a : b;
            }
        }
    }
}

// Fully unrolled network (E <= 8): every stage's lane exchange and
// direction are compile-time, so a stage is exchanges + compare + selects.
template <int E, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_cross_levels(uint64_t (&v)[E], int l)
{
    if constexpr (STRIDE >= E && STRIDE >= 1) {
        const int e = l * E;
        const bool keep_max = ((e & STRIDE) == 0) == ((e & SIZE) == 0);
        cross_stage<STRIDE / E, E>(v, keep_max);
        bitonic_cross_levels<E, SIZE, STRIDE / 2>(v, l);
    }
}

template <int E, int SIZE>
__device__ __forceinline__ void bitonic_levels(uint64_t (&v)[E], int l)
{
    bitonic_cross_levels<E, SIZE, SIZE / 2>(v, l);
    bitonic_in_lane_fixed<E, SIZE>(v, l);
    if constexpr (SIZE < kWave * E)
        bitonic_levels<E, SIZE * 2>(v, l);
}

template <int E>
__device__ __forceinline__ void bitonic_sort_desc(uint64_t (&v)[E], int l)
{
    if constexpr (E <= 8) {
        bitonic_levels<E, 2>(v, l);
    } else {
#pragma unroll 1
        for (int size = 2; size <= kWave * E; size <<= 1) {
#pragma unroll 1
            for (int stride = size >> 1; stride >= E; stride >>= 1) {
                const int e = l * E;
                const bool keep_max = ((e & stride) == 0) == ((e & size) == 0);
                switch (stride / E) {
                case 1: cross_stage<1, E>(v, keep_max); break;
                case 2: cross_stage<2, E>(v, keep_max); break;
                case 4: cross_stage<4, E>(v, keep_max); break;
                case 8: cross_stage<8, E>(v, keep_max); break;
                case 16: cross_stage<16, E>(v, keep_max); break;
                default: cross_stage<32, E>(v, keep_max); break;
                }
            }
            bitonic_in_lane<E>(v, size, l);
        }
    }
}

// Sort the n pairs key/ent[0..n) and write out[0..k): entries, then -1.
template <int E, typename EntT>
__device__ __forceinline__ void sort_and_write(const uint32_t *key, const EntT *ent, int n, int k, int32_t *out)
{
    const int l = opaque_lane();
    uint64_t v[E];
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int e = l * E + r;
        // ~entry in the low half: among equal keys the lower entry sorts first.
        v[r] = (e < n) ? (((uint64_t)key[e] << 32) | (uint32_t)~(uint32_t)ent[e]) : 0ull;
    }
    bitonic_sort_desc<E>(v, l);
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int e = l * E + r;
        if (e < k)
            out[e] = (e < n) ? (int32_t)~(uint32_t)v[r] : -1;
    }
    for (int e = kWave * E + l; e < k; e += kWave)
        out[e] = -1;
}

// ---------------------------------------------------------------------------
// Faster sort for buffers in which equal keys appear in entry order (every
// buffer the top-k code sorts has that property): sort 32-bit composites
// ((key - kmin) >> shift) << PB | (64E-1 - position) descending, where PB bits
// hold the position and shift drops just enough low key bits to fit.  A
// compare-exchange is then one v_med3_u32 against an all-ones / all-zeros
// selector.  Equal keys order by position, i.e. by entry.  If dropping bits
// made two different keys look equal, the result is discarded and the exact
// 64-bit sort runs instead.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t med3u(uint32_t a, uint32_t b, uint32_t c)
{
    uint32_t r;
    __asm__("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Compare-exchange of element r with the same element of lane l ^ LX for
// LX = 16 or 32, two elements (r, r + 1) at a time: one lane swap between the
// two registers leaves, in every lane, both values of one of the two pairs
// (element r's pair in the lanes whose LX bit is clear, element r + 1's in
// the others); both results are computed in that lane and a second swap puts
// them back.  The lane holding a pair computes its own result into the
// register of its own element, and its partner's into the other.
template <int LX>
__device__ __forceinline__ void swap_halves(uint32_t &x, uint32_t &y)
{
    static_assert(LX == 16 || LX == 32, "lane swaps exist for distances 16 and 32");
    const auto sw = LX == 16 ? __builtin_amdgcn_permlane16_swap(x, y, false, false)
                             : __builtin_amdgcn_permlane32_swap(x, y, false, false);
    x = sw[0];
    y = sw[1];
}

// s_first selects the larger value for the first of the two values a lane
// holds after the swap: in lanes whose LX bit is set that pair is the
// partner's element r + 1 (first) and this lane's (second), so the results
// trade places.
template <int E, int LX>
__device__ __forceinline__ void cross_stage32_swapped(uint32_t (&v)[E], uint32_t s_first)
{
    static_assert(E % 2 == 0, "elements are exchanged in pairs");
#pragma unroll
    for (int r = 0; r < E; r += 2)
        swap_halves<LX>(v[r], v[r + 1]);
#pragma unroll
    for (int r = 0; r < E; r += 2) {
        const uint32_t x = v[r], y = v[r + 1];
        v[r] = med3u(x, y, s_first);
        v[r + 1] = med3u(x, y, ~s_first);
    }
#pragma unroll
    for (int r = 0; r < E; r += 2)
        swap_halves<LX>(v[r], v[r + 1]);
}

template <int E, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic32_cross_levels(uint32_t (&v)[E], int l)
{
    if constexpr (STRIDE >= E && STRIDE >= 1) {
        // lane l keeps the larger value when bit STRIDE of l * E equals bit
        // SIZE of it, i.e. lane bits STRIDE / E and SIZE / E
        constexpr int LX = STRIDE / E;
        constexpr uint64_t keep = ~(lanes_bit_clear(LX) ^ lanes_bit_clear(SIZE / E));
        if constexpr ((LX == 16 || LX == 32) && E % 2 == 0) {
            // a lane with bit LX set computes its partner's result first
            cross_stage32_swapped<E, LX>(v, lane_sel(keep ^ ~lanes_bit_clear(LX)));
        } else {
            const uint32_t sel = lane_sel(keep);
            // all exchanges first, then the compare-exchanges, so no
            // exchange waits on the result just computed
            uint32_t o[E];
#pragma unroll
            for (int r = 0; r < E; ++r)
                o[r] = lane_xor_u32<LX>(v[r]);
#pragma unroll
            for (int r = 0; r < E; ++r)
                v[r] = med3u(v[r], o[r], sel);
        }
        bitonic32_cross_levels<E, SIZE, STRIDE / 2>(v, l);
    }
}

template <int E, int SIZE>
__device__ __forceinline__ void bitonic32_in_lane(uint32_t (&v)[E], int l)
{
    // first element of a pair takes the max when its block sorts descending
    // (bit SIZE of l * E clear: lane bit SIZE / E)
    const uint32_t sel = SIZE >= E ? lane_sel(lanes_bit_clear(SIZE >= E ? SIZE / E : 1)) : 0u;
#pragma unroll
    for (int stride = (SIZE / 2 < E / 2 ? SIZE / 2 : E / 2); stride >= 1; stride >>= 1) {
#pragma unroll
        for (int r = 0; r < E; ++r) {
            if ((r & stride) == 0) {
                const uint32_t a = v[r], b = v[r + stride];
                if constexpr (SIZE >= E) {
                    v[r] = med3u(a, b, sel);
                    v[r + stride] = med3u(a, b, ~sel);
                } else if ((r & SIZE) == 0) {
                    v[r] = max(a, b);
                    v[r + stride] = min(a, b);
                } else {
                    v[r] = min(a, b);
                    v[r + stride] = max(a, b);
                }
            }
        }
    }
}

template <int E, int SIZE>
__device__ __forceinline__ void bitonic32_levels(uint32_t (&v)[E], int l)
{
    bitonic32_cross_levels<E, SIZE, SIZE / 2>(v, l);
    bitonic32_in_lane<E, SIZE>(v, l);
    if constexpr (SIZE < kWave * E)
        bitonic32_levels<E, SIZE * 2>(v, l);
}

// Value of v in lane (lane + 1); lane 63 gets its own value.
__device__ __forceinline__ uint32_t from_next_lane(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x130, 0xF, 0xF, false); // wave_shl:1
}

// Returns false (and writes nothing) when the truncated composites cannot
// order the buffer exactly.  With kRange the caller passes bounds lo <= every
// key <= hi of key[0..n) (wave-uniform) instead of having them reduced here.
template <int E, typename EntT, bool kRange = false>
__device__ __forceinline__ bool sort_and_write_fast(const uint32_t *key, const EntT *ent, int n, int k, int32_t *out,
                                                    uint32_t lo = 0u, uint32_t hi = 0u)
{
    constexpr int PB = (E == 1) ? 6 : (E == 2) ? 7 : (E == 4) ? 8 : 9;
    static_assert((kWave * E) == (1 << PB), "position bits");
    constexpr uint32_t kPosMask = (1u << PB) - 1u;
    const int l = opaque_lane();
    uint32_t kr[E];
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int e = l * E + r;
        kr[r] = e < n ? key[e] : 0u;
        mn = e < n ? min(mn, kr[r]) : mn;
        mx = max(mx, kr[r]);
    }
    uint32_t kmin = lo, span = hi - lo;
    if constexpr (!kRange) {
        mn = min(mn, lane_xor_u32<1>(mn));
        mx = max(mx, lane_xor_u32<1>(mx));
        mn = min(mn, lane_xor_u32<2>(mn));
        mx = max(mx, lane_xor_u32<2>(mx));
        mn = min(mn, lane_xor_u32<4>(mn));
        mx = max(mx, lane_xor_u32<4>(mx));
        mn = min(mn, lane_xor_u32<8>(mn));
        mx = max(mx, lane_xor_u32<8>(mx));
        mn = min(mn, lane_xor_u32<16>(mn));
        mx = max(mx, lane_xor_u32<16>(mx));
        mn = min(mn, lane_xor_u32<32>(mn));
        mx = max(mx, lane_xor_u32<32>(mx));
        kmin = uniform_u(mn);
        span = uniform_u(mx) - kmin;
    }
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    const int shift = bits > 32 - PB ? bits - (32 - PB) : 0;
    uint32_t c[E];
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int e = l * E + r;
        // empty slots are 0.  A valid composite is 0 only for the element at
        // e = 64E-1 with a key in the lowest bucket, and then n = 64E and no
        // slot is empty, so after the sort the n valid elements hold sorted
        // positions 0 .. n-1 in every case.
        c[r] = e < n ? (((kr[r] - kmin) >> shift) << PB) | (kPosMask - (uint32_t)e) : 0u;
    }
    bitonic32_levels<E, 2>(c, l);
    if (shift > 0) {
        // adjacent elements whose truncated keys are equal must have equal
        // keys; a pair takes part when both its sorted positions are below n
        bool bad = false;
        const uint32_t next0 = from_next_lane(c[0]);
#pragma unroll
        for (int r = 0; r < E; ++r) {
            const uint32_t a = c[r], b = (r + 1 < E) ? c[r + 1] : next0;
            const bool pair_in = l * E + r + 1 < n;
            if (pair_in && (a >> PB) == (b >> PB))
                bad = bad || key[kPosMask - (a & kPosMask)] != key[kPosMask - (b & kPosMask)];
        }
        if (ballot(bad) != 0ull)
            return false;
    }
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int e = l * E + r;
        if (e < k)
            out[e] = (e < n) ? (int32_t)ent[kPosMask - (c[r] & kPosMask)] : -1;
    }
    for (int e = kWave * E + l; e < k; e += kWave)
        out[e] = -1;
    return true;
}

// sort_pairs_and_write for n pairs whose keys all lie in [lo, hi]
// (wave-uniform bounds known to the caller).
template <typename EntT>
__device__ __forceinline__ void sort_pairs_in_range_and_write(const uint32_t *key, const EntT *ent, int n, int k,
                                                              int32_t *out, uint32_t lo, uint32_t hi)
{
    wave_lds_fence();
    if (n <= 64) {
        if (!sort_and_write_fast<1, EntT, true>(key, ent, n, k, out, lo, hi))
            sort_and_write<1, EntT>(key, ent, n, k, out);
    } else if (n <= 128) {
        if (!sort_and_write_fast<2, EntT, true>(key, ent, n, k, out, lo, hi))
            sort_and_write<2, EntT>(key, ent, n, k, out);
    } else if (n <= 256) {
        if (!sort_and_write_fast<4, EntT, true>(key, ent, n, k, out, lo, hi))
            sort_and_write<4, EntT>(key, ent, n, k, out);
    } else if (n <= 512) {
        if (!sort_and_write_fast<8, EntT, true>(key, ent, n, k, out, lo, hi))
            sort_and_write<8, EntT>(key, ent, n, k, out);
    } else if (n <= 1024) {
        sort_and_write<16, EntT>(key, ent, n, k, out);
    } else {
        sort_and_write<32, EntT>(key, ent, n, k, out);
    }
}

template <typename EntT>
__device__ __forceinline__ void sort_pairs_and_write(const uint32_t *key, const EntT *ent, int n, int k, int32_t *out)
{
    wave_lds_fence();
    if (n <= 64) {
        if (!sort_and_write_fast<1, EntT>(key, ent, n, k, out))
            sort_and_write<1, EntT>(key, ent, n, k, out);
    } else if (n <= 128) {
        if (!sort_and_write_fast<2, EntT>(key, ent, n, k, out))
            sort_and_write<2, EntT>(key, ent, n, k, out);
    } else if (n <= 256) {
        if (!sort_and_write_fast<4, EntT>(key, ent, n, k, out))
            sort_and_write<4, EntT>(key, ent, n, k, out);
    } else if (n <= 512) {
        if (!sort_and_write_fast<8, EntT>(key, ent, n, k, out))
            sort_and_write<8, EntT>(key, ent, n, k, out);
    } else if (n <= 1024) {
        sort_and_write<16, EntT>(key, ent, n, k, out);
    } else {
        sort_and_write<32, EntT>(key, ent, n, k, out);
    }
}

// Final selection of the row into out[0..k) (global memory).
template <typename EntT>
__device__ __forceinline__ void topk_finish(TopKRow<EntT> &t, int32_t *out)
{
    topk_reduce(t);
    sort_pairs_and_write(t.key, t.ent, t.count, t.k, out);
}

// Histogram of the register-held keys kr[] (0 = no key; every buffered key
// is above the key of -inf, so never 0) that lie in [base, base + span], by
// (key - base) >> shift, then the bucket holding the kk-th largest of them
// (find_digit).  `inb` receives that bucket's count.
template <int NR>
__device__ __forceinline__ int bucket_of_kth_regs(const uint32_t (&kr)[NR], uint32_t base, uint32_t span, int shift,
                                                  int kk, uint32_t *hist, int &above, int &inb)
{
    for (int b = lane(); b < 256; b += kWave)
        hist[b] = 0u;
    wave_lds_fence();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        // an empty slot (0) wraps to 0 - base > span: base >= 1
        const uint32_t off = kr[r] - base;
        if (off <= span)
            atomicAdd(&hist[off >> shift], 1u);
    }
    wave_lds_fence();
    const int d = find_digit(hist, kk, above);
    inb = uniform((int)hist[d]);
    wave_lds_fence();
    return d;
}

// Final selection for buffers of at most 64*NR pairs, with the keys held in
// registers: lane l holds the pairs at 256*m + 4*l + c (m < NR/4, c < 4).
// One LDS read of every key and entry, range-adaptive histogram passes from
// registers until the k-th key's bucket holds at most 64 keys, that bucket
// sorted in registers, then the k winners (keys above T, and the earliest
// ties) written back to the front of the buffer for the final sort.
template <int NR, typename EntT>
__device__ __forceinline__ void topk_finish_regs(TopKRow<EntT> &t, int32_t *out)
{
    static_assert(NR % 4 == 0, "four pairs per lane per group");
    const int n = t.count, k = t.k, l = opaque_lane();
    wave_lds_fence();
    if (n <= k) {
        sort_pairs_and_write(t.key, t.ent, n, k, out);
        return;
    }
    uint32_t kr[NR];
    EntT er[NR];
#pragma unroll
    for (int m = 0; m < NR / 4; ++m) {
        // i0 < n <= cap, all multiples of 4: the group lies in the buffer
        const int i0 = 256 * m + 4 * l;
        const bool in = i0 < n;
        const u32x4 q = in ? *reinterpret_cast<const u32x4 *>(t.key + i0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            kr[4 * m + c] = i0 + c < n ? q[c] : 0u;
            er[4 * m + c] = in ? t.ent[i0 + c] : (EntT)0;
        }
    }
    // key range of the valid keys
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        mn = min(mn, kr[r] != 0u ? kr[r] : 0xFFFFFFFFu);
        mx = max(mx, kr[r]);
    }
    mn = min(mn, lane_xor_u32<1>(mn));
    mx = max(mx, lane_xor_u32<1>(mx));
    mn = min(mn, lane_xor_u32<2>(mn));
    mx = max(mx, lane_xor_u32<2>(mx));
    mn = min(mn, lane_xor_u32<4>(mn));
    mx = max(mx, lane_xor_u32<4>(mx));
    mn = min(mn, lane_xor_u32<8>(mn));
    mx = max(mx, lane_xor_u32<8>(mx));
    mn = min(mn, lane_xor_u32<16>(mn));
    mx = max(mx, lane_xor_u32<16>(mx));
    mn = min(mn, lane_xor_u32<32>(mn));
    mx = max(mx, lane_xor_u32<32>(mx));
    const uint32_t kmax = uniform_u(mx);
    uint32_t base = uniform_u(mn), span = kmax - base;
    int kk = k;
    uint32_t T = base;
    int ties_keep = 0;
    bool resolved = false;
#pragma unroll 1
    while (span != 0u) {
        const int bits = 32 - __builtin_clz(span);
        const int shift = bits > 8 ? bits - 8 : 0;
        int above, inb;
        const uint32_t d = (uint32_t)bucket_of_kth_regs<NR>(kr, base, span, shift, kk, t.hist, above, inb);
        kk -= above;
        base += d << shift;
        if (shift == 0)
            break;
        span = min(span - (d << shift), (1u << shift) - 1u);
        if (inb <= kWave) {
            // gather the bucket's keys (any order), one per lane, and sort them
            int cnt = 0;
#pragma unroll
            for (int r = 0; r < NR; ++r)
                cnt += (kr[r] - base <= span) ? 1 : 0;
            int pos = wave_exclusive_sum(cnt);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                if (kr[r] - base <= span)
                    t.hist[pos++] = kr[r];
            }
            wave_lds_fence();
            const uint32_t x = l < inb ? t.hist[l] : 0u;
            const uint32_t sx = sort_u32_desc(x, l);
            T = uniform_u((uint32_t)read_lane((int)sx, kk - 1));
            ties_keep = kk - popc64(ballot(sx > T));
            resolved = true;
            wave_lds_fence();
            break;
        }
    }
    if (!resolved) {
        T = base;
        ties_keep = kk;
    }
    // winners: keys > T and the first ties_keep keys == T, placed at the
    // front in buffer order.  Slot c of lane l in group m is buffer entry
    // 256m + 4l + c, so within a group the pairs of lower lanes come first
    // (counted from four ballots), then this lane's in c order.
    int g_base = 0, e_base = 0;
#pragma unroll
    for (int m = 0; m < NR / 4; ++m) {
        uint64_t beq[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            beq[c] = ballot(kr[4 * m + c] == T);
        int e = e_base;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            e += rank_below(beq[c]);
        bool win[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t x = kr[4 * m + c];
            win[c] = x > T || (x == T && e < ties_keep);
            e += x == T ? 1 : 0;
        }
        uint64_t bw[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            bw[c] = ballot(win[c]);
        int p = g_base;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            p += rank_below(bw[c]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int r = 4 * m + c;
            if (win[c]) {
                t.key[p] = kr[r];
                t.ent[p] = er[r];
                ++p;
            }
        }
        g_base += popc64(bw[0]) + popc64(bw[1]) + popc64(bw[2]) + popc64(bw[3]);
        e_base += popc64(beq[0]) + popc64(beq[1]) + popc64(beq[2]) + popc64(beq[3]);
    }
    t.count = k;
    t.tau = T;
    sort_pairs_in_range_and_write(t.key, t.ent, k, k, out, T, kmax);
}

// ---------------------------------------------------------------------------
// Block-level finish.  Wave w of NW holds key/ent[w*cap .. w*cap + cnt[w]) in
// LDS, each already reduced to at most k pairs, segments in entry order.  All
// NW waves of the workgroup call this together.  `hist` is 256 shared words,
// `cnt` NW+2 shared words, `sel_key`/`sel_ent` k shared words each.
// ---------------------------------------------------------------------------
template <int NW>
__device__ __forceinline__ void block_select_sort(uint32_t *key, uint32_t *ent, int cap, int my_count, int k,
                                                  uint32_t *hist, int *cnt, uint32_t *sel_key, uint32_t *sel_ent,
                                                  int32_t *out)
{
    const int wv = threadIdx.x / kWave, l = lane();
    uint32_t *mk = key + wv * cap;
    uint32_t *me = ent + wv * cap;
    if (l == 0)
        cnt[wv] = my_count;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        total += cnt[w];

    uint32_t T = 0u;
    int kk = 0;
    const bool select = total > k;
    if (select) {
        uint32_t prefix = 0u, mask = 0u;
        kk = k;
#pragma unroll 1
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int b = threadIdx.x; b < 256; b += NW * kWave)
                hist[b] = 0u;
            __syncthreads();
            for (int i = l; i < my_count; i += kWave) {
                const uint32_t kv = mk[i];
                if ((kv & mask) == prefix)
                    atomicAdd(&hist[(kv >> shift) & 0xFFu], 1u);
            }
            __syncthreads();
            if (wv == 0) {
                int above;
                const int digit = find_digit(hist, kk, above);
                if (l == 0) {
                    cnt[NW] = digit;
                    cnt[NW + 1] = above;
                }
            }
            __syncthreads();
            kk -= cnt[NW + 1];
            prefix |= (uint32_t)cnt[NW] << shift;
            mask |= 0xFFu << shift;
            __syncthreads();
        }
        T = prefix;
    }
    // per-wave counts of winners above T and of ties, for ordered placement
    int gt = 0, eq = 0;
    for (int i = l; i < my_count; i += kWave) {
        const uint32_t kv = mk[i];
        gt += (!select || kv > T) ? 1 : 0;
        eq += (select && kv == T) ? 1 : 0;
    }
    gt = wave_exclusive_sum(gt) + gt; // inclusive: last lane has the wave total
    eq = wave_exclusive_sum(eq) + eq;
    if (l == kWave - 1) {
        hist[wv] = (uint32_t)gt;
        hist[NW + wv] = (uint32_t)eq;
    }
    __syncthreads();
    int gt_before = 0, eq_before = 0, gt_total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        gt_before += (w < wv) ? (int)hist[w] : 0;
        eq_before += (w < wv) ? (int)hist[NW + w] : 0;
        gt_total += (int)hist[w];
    }
    const int n_sel = select ? k : total;
    // winners above T go first (in entry order), then the earliest ties
    int gpos = gt_before, epos = eq_before;
#pragma unroll 1
    for (int base = 0; base < my_count; base += kWave) {
        const int i = base + l;
        const bool in = i < my_count;
        const uint32_t kv = in ? mk[i] : 0u;
        const uint32_t ev = in ? me[i] : 0u;
        const bool g = in && (!select || kv > T);
        const bool e = in && select && kv == T;
        const uint64_t bg = ballot(g), be = ballot(e);
        if (g) {
            const int p = gpos + rank_below(bg);
            sel_key[p] = kv;
            sel_ent[p] = ev;
        }
        if (e) {
            const int r = epos + rank_below(be);
            if (r < kk) {
                sel_key[gt_total + r] = kv;
                sel_ent[gt_total + r] = ev;
            }
        }
        gpos += popc64(bg);
        epos += popc64(be);
    }
    __syncthreads();
    if (wv == 0)
        sort_pairs_and_write(sel_key, sel_ent, n_sel, k, out);
}

} // namespace csa
