// Exact per-row top-k, run by one wave over a stream of (key, entry) pairs that
// arrive in increasing entry order, 64 at a time.
//
// The wave keeps a candidate buffer of `cap` pairs in LDS and a threshold
// tau: a pair may enter only if its key is > tau.  When the buffer would
// overflow, a radix select finds T, the k-th largest key in the buffer, and an
// order-preserving compaction keeps every key > T plus the earliest keys == T
// up to k pairs; tau becomes T.  A later pair with key <= T can never make the
// top k: k kept pairs beat it (larger key, or equal key and lower entry).  At
// the end the same select leaves exactly min(k, count) pairs, which a bitonic
// sort orders by (key descending, entry ascending).
//
// Keys are score_key() images of fp32 scores, so key order is score order and
// -0 ties with +0.
#pragma once

#include "csa_device.hpp"
#include "csa_launch.hpp"

namespace csa {

struct TopKRow {
    uint32_t *key; // LDS [cap]
    uint32_t *ent; // LDS [cap]
    uint32_t *hist; // LDS [256], scratch of the owning wave
    int cap;       // >= k + 64
    int k;
    int count;     // wave-uniform
    uint32_t tau;  // wave-uniform
};

__device__ __forceinline__ void topk_init(TopKRow &t, uint32_t *key, uint32_t *ent, uint32_t *hist, int cap, int k)
{
    t.key = key;
    t.ent = ent;
    t.hist = hist;
    t.cap = cap;
    t.k = k;
    t.count = 0;
    t.tau = kKeyNegInf;
}

// Radix select over key[0..count), count > k: the k-th largest key T, and how
// many keys equal to T belong to the top k (the earliest ones in buffer order).
__device__ __forceinline__ void radix_select(const uint32_t *key, int count, int k, uint32_t *hist, uint32_t &T,
                                             int &ties_keep)
{
    const int l = lane();
    uint32_t prefix = 0u, mask = 0u;
    int kk = k;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int bin = l; bin < 256; bin += kWave)
            hist[bin] = 0u;
        wave_lds_fence();
        for (int i = l; i < count; i += kWave) {
            const uint32_t kv = key[i];
            if ((kv & mask) == prefix)
                atomicAdd(&hist[(kv >> shift) & 0xFFu], 1u);
        }
        wave_lds_fence();
        // lane l owns bins 255-4l, 254-4l, 253-4l, 252-4l (descending).
        int h[4], tot = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            h[r] = (int)hist[255 - 4 * l - r];
            tot += h[r];
        }
        int cum = wave_exclusive_sum(tot);
        int found = -1, above = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (found < 0 && cum < kk && kk <= cum + h[r]) {
                found = 255 - 4 * l - r;
                above = cum;
            }
            cum += h[r];
        }
        const uint64_t bal = ballot(found >= 0);
        const int src = bal ? (int)__builtin_ctzll(bal) : 0;
        const int digit = read_lane(found, src);
        kk -= read_lane(above, src);
        prefix |= (uint32_t)(digit & 0xFF) << shift;
        mask |= 0xFFu << shift;
        wave_lds_fence();
    }
    T = prefix;
    ties_keep = kk;
}

// Keep keys > T and the first ties_keep keys == T, in place and in order.
// Returns the new count.
__device__ __forceinline__ int compact_keep(uint32_t *key, uint32_t *ent, int count, uint32_t T, int ties_keep)
{
    int out = 0, ties = 0;
#pragma unroll 1
    for (int base = 0; base < count; base += kWave) {
        const int i = base + lane();
        const bool in = i < count;
        const uint32_t kv = in ? key[i] : 0u;
        const uint32_t ev = in ? ent[i] : 0u;
        const bool eq = in && kv == T;
        const uint64_t beq = ballot(eq);
        const bool keep = (in && kv > T) || (eq && ties + rank_below(beq) < ties_keep);
        ties += popc64(beq);
        const uint64_t bk = ballot(keep);
        if (keep) {
            const int pos = out + rank_below(bk);
            key[pos] = kv;
            ent[pos] = ev;
        }
        out += popc64(bk);
    }
    wave_lds_fence();
    return out;
}

// Offer one pair per lane; lanes must hold increasing entries.
__device__ __forceinline__ void topk_push(TopKRow &t, uint32_t kv, uint32_t entry, bool valid)
{
    bool pass = valid && kv > t.tau;
    uint64_t bal = ballot(pass);
    int n = popc64(bal);
    if (t.count + n > t.cap) {
        uint32_t T;
        int keep;
        radix_select(t.key, t.count, t.k, t.hist, T, keep);
        t.count = uniform(compact_keep(t.key, t.ent, t.count, T, keep));
        t.tau = uniform_u(T);
        pass = valid && kv > t.tau;
        bal = ballot(pass);
        n = popc64(bal);
    }
    if (pass) {
        const int pos = t.count + rank_below(bal);
        t.key[pos] = kv;
        t.ent[pos] = entry;
    }
    t.count += n;
    wave_lds_fence();
}

// In-register stages (partner in the same lane) of one bitonic merge level.
template <int E>
__device__ __forceinline__ void bitonic_in_lane(uint64_t (&v)[E], int size, int l)
{
#pragma unroll
    for (int stride = E / 2; stride >= 1; stride >>= 1) {
        if (stride < size) {
#pragma unroll
            for (int r = 0; r < E; ++r) {
                if ((r & stride) == 0) {
                    const int e = l * E + r;
                    const bool desc = (e & size) == 0;
                    const uint64_t a = v[r], b = v[r + stride];
                    const bool sw = desc ? (a < b) : (a > b);
                    v[r] = sw ? b : a;
                    v[r + stride] = sw ? a : b;
                }
            }
        }
    }
}

// Sort the 64*E values held by the wave (lane l holds elements l*E .. l*E+E-1)
// in descending order.
template <int E>
__device__ __forceinline__ void bitonic_sort_desc(uint64_t (&v)[E])
{
    const int l = lane();
#pragma unroll 1
    for (int size = 2; size <= kWave * E; size <<= 1) {
#pragma unroll 1
        for (int stride = size >> 1; stride >= E; stride >>= 1) {
            const int lx = stride / E;
#pragma unroll
            for (int r = 0; r < E; ++r) {
                const int e = l * E + r;
                const uint64_t o = shfl_xor_u64(v[r], lx);
                const bool keep_max = ((e & stride) == 0) == ((e & size) == 0);
                const uint64_t mx = v[r] > o ? v[r] : o;
                const uint64_t mn = v[r] > o ? o : v[r];
                v[r] = keep_max ? mx : mn;
            }
        }
        bitonic_in_lane<E>(v, size, l);
    }
}

// Sort the n selected pairs and write out[0..k): entries, then -1 padding.
template <int E>
__device__ __forceinline__ void sort_and_write(const uint32_t *key, const uint32_t *ent, int n, int k, int32_t *out)
{
    const int l = lane();
    uint64_t v[E];
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int e = l * E + r;
        // ~entry in the low half: among equal keys the lower entry sorts first.
        v[r] = (e < n) ? (((uint64_t)key[e] << 32) | (uint32_t)~ent[e]) : 0ull;
    }
    bitonic_sort_desc<E>(v);
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int e = l * E + r;
        if (e < k)
            out[e] = (e < n) ? (int32_t)~(uint32_t)v[r] : -1;
    }
    for (int e = kWave * E + l; e < k; e += kWave)
        out[e] = -1;
}

// Final selection of the row into out[0..k) (global memory).
__device__ __forceinline__ void topk_finish(TopKRow &t, int32_t *out)
{
    int n = t.count;
    if (n > t.k) {
        uint32_t T;
        int keep;
        radix_select(t.key, n, t.k, t.hist, T, keep);
        n = uniform(compact_keep(t.key, t.ent, n, T, keep));
    }
    if (n <= 64)
        sort_and_write<1>(t.key, t.ent, n, t.k, out);
    else if (n <= 128)
        sort_and_write<2>(t.key, t.ent, n, t.k, out);
    else if (n <= 256)
        sort_and_write<4>(t.key, t.ent, n, t.k, out);
    else if (n <= 512)
        sort_and_write<8>(t.key, t.ent, n, t.k, out);
    else if (n <= 1024)
        sort_and_write<16>(t.key, t.ent, n, t.k, out);
    else
        sort_and_write<32>(t.key, t.ent, n, t.k, out);
}

} // namespace csa
