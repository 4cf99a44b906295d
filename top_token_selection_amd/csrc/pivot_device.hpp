// pivot_device.hpp -- device building blocks of the PIVOT indexer (gfx950).
//
// * Ranking keys: a float32 score maps to a uint32 whose unsigned order is
//   the score order (-0.0 folded onto +0.0). The total order of the method
//   (larger score first, equal scores -> smaller key index first) becomes
//   "larger key first, then smaller index".
// * Group<NW>: NW wavefronts (64 lanes each) that cooperate on one selection
//   through a private LDS area; NW == 1 needs no workgroup barrier.
// * Selector: exact top-m selection by range-bucket radix narrowing. Each
//   pass histograms the keys still in play into NB buckets spanning exactly
//   their current [lo, hi] range, keeps the bucket holding the m-th largest
//   and repeats on it; equal keys at the boundary are resolved by key index
//   with the same narrowing on ~index. Then a bucket sort orders the
//   selected elements (score descending, index ascending).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pivot {

typedef uint16_t bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// --------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// Round-to-nearest-even float32 -> bf16 (finite values).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float load_f32(const float *p) { return *p; }
__device__ __forceinline__ float load_f32(const bf16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_from_f32(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_from_f32(bf16_t *p, float v) { *p = f32_to_bf16(v); }

// Order-preserving uint32 image of a score.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ int bit_width(uint32_t x) { return x ? 32 - __clz((int)x) : 0; }

// ------------------------------------------------------------ wavefronts

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Cross-lane steps use DPP (data-parallel primitives of the VALU): row_shr:n
// (row_shl:n) gives lane l the value of lane l - n (l + n) of its row of 16
// lanes, wave_shr:1 (wave_shl:1) that of lane l - 1 (l + 1) of the whole
// wavefront, row_bcast:15 / row_bcast:31 carry lane
// 15 of a row into the next row / lane 31 into rows 2 and 3. A lane with no
// source (or in a row left out by the row mask) gets `old`.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
// v of another lane by DPP, 0 where the source lane is outside the row
// (bound_ctrl): there is no old value to keep, so no register is set first
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_zero(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;
constexpr int DPP_ROW_SHL4 = 0x104;
constexpr int DPP_WAVE_SHL1 = 0x130, DPP_WAVE_SHR1 = 0x138;
constexpr int DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

// op over lanes 0..l for every lane l (inclusive scan); lane 63 ends with
// the op over the whole wavefront. `id` is op's identity.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan_op(uint32_t v, uint32_t id, Op op) {
    v = op(v, dpp_u32<DPP_ROW_SHR1>(id, v));
    v = op(v, dpp_u32<DPP_ROW_SHR2>(id, v));
    v = op(v, dpp_u32<DPP_ROW_SHR4>(id, v));
    v = op(v, dpp_u32<DPP_ROW_SHR8>(id, v));
    v = op(v, dpp_u32<DPP_ROW_BCAST15, 0xA>(id, v));
    v = op(v, dpp_u32<DPP_ROW_BCAST31, 0xC>(id, v));
    return v;
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
    v = wave_scan_op(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return min(a, b); });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = wave_scan_op(v, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    v = wave_scan_op(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    return wave_scan_op(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// LDS ordering point for a single wavefront working in its private area.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
}

// NW wavefronts cooperating through LDS. `tid` runs over 0 .. 64*NW-1;
// `red` is LDS scratch of at least 2*NW+8 words private to the group.
template <int NW>
struct Group {
    static constexpr int NT = 64 * NW;
    int tid;
    uint32_t *red;

    __device__ __forceinline__ void sync() const {
        if constexpr (NW == 1) wave_lds_sync();
        else __syncthreads();
    }
    __device__ __forceinline__ int wave() const { return tid >> 6; }

    __device__ __forceinline__ uint32_t reduce_min(uint32_t v) const {
        v = wave_min(v);
        if constexpr (NW == 1) return v;
        if (lane_id() == 0) red[wave()] = v;
        sync();
        uint32_t r = red[0];
        for (int w = 1; w < NW; ++w) r = min(r, red[w]);
        sync();
        return r;
    }
    __device__ __forceinline__ uint32_t reduce_max(uint32_t v) const {
        v = wave_max(v);
        if constexpr (NW == 1) return v;
        if (lane_id() == 0) red[wave()] = v;
        sync();
        uint32_t r = red[0];
        for (int w = 1; w < NW; ++w) r = max(r, red[w]);
        sync();
        return r;
    }
    __device__ __forceinline__ uint32_t reduce_sum(uint32_t v) const {
        v = wave_sum(v);
        if constexpr (NW == 1) return v;
        if (lane_id() == 0) red[wave()] = v;
        sync();
        uint32_t r = 0;
        for (int w = 0; w < NW; ++w) r += red[w];
        sync();
        return r;
    }
    // Exclusive prefix sum over the group in thread order.
    __device__ __forceinline__ uint32_t excl_scan(uint32_t v) const {
        uint32_t inc = wave_incl_scan(v);
        if constexpr (NW == 1) return inc - v;
        if (lane_id() == 63) red[wave()] = inc;
        sync();
        uint32_t base = 0;
        for (int w = 0; w < wave(); ++w) base += red[w];
        sync();
        return base + inc - v;
    }
};

// Selection rule: element (key, idx) is selected iff
//   key > T  or  (key == T and ~idx >= I).
// {0, 0} selects everything.
struct Rule {
    uint32_t T;
    uint32_t I;
    __device__ __forceinline__ bool sel(uint32_t key, uint32_t idx) const {
        return key > T || (key == T && (~idx) >= I);
    }
};

// Exact top-m selection and ordering for one group of NW wavefronts.
// `hist` is LDS of NB = 2^LOG2NB words private to the group; `vars` is 4
// private LDS words. Element streams are supplied by the caller as
//   fe(f)   -- calls f(key, payload) for each element the thread owns,
//   idx(p)  -- key index of a payload.
template <int NW, int LOG2NB>
struct Selector {
    static constexpr int NB = 1 << LOG2NB;
    static constexpr int NT = 64 * NW;
    static_assert(NB % NT == 0, "histogram must split evenly over the group");
    static constexpr int BPT = NB / NT;

    Group<NW> G;
    uint32_t *hist;
    uint32_t *vars;

    __device__ __forceinline__ void clear_hist() const {
        for (int b = G.tid; b < NB; b += NT) hist[b] = 0;
    }

    // Bucket holding the need-th largest element: bins are scanned from the
    // top (largest keys) down. Returns the bucket, the count above it and
    // its own count.
    __device__ __forceinline__ void crossing(uint32_t need, uint32_t &b_out, uint32_t &above,
                             uint32_t &cnt) const {
        if (G.tid == 0) {
            vars[0] = 0;
            vars[1] = 0;
            vars[2] = 0;
        }
        uint32_t loc = 0;
        for (int i = 0; i < BPT; ++i) loc += hist[NB - 1 - (G.tid * BPT + i)];
        uint32_t pre = G.excl_scan(loc);
        if (pre < need && need <= pre + loc) {
            uint32_t cum = pre;
            for (int i = 0; i < BPT; ++i) {
                uint32_t bb = NB - 1 - (G.tid * BPT + i);
                uint32_t h = hist[bb];
                if (cum + h >= need) {
                    vars[0] = bb;
                    vars[1] = cum;
                    vars[2] = h;
                    break;
                }
                cum += h;
            }
        }
        G.sync();
        b_out = vars[0];
        above = vars[1];
        cnt = vars[2];
        G.sync();
    }

    // Narrow [lo, hi] until the need-th largest value is pinned. ext(key,
    // payload, valid, k) maps an element to its ranking value k. Result:
    // `whole` -> the selection is exactly {k >= T}; otherwise it is
    // {k > T} plus `rem` of the elements with k == T.
    template <class FE, class EXT>
    __device__ __forceinline__ void narrow(FE fe, EXT ext, uint32_t lo, uint32_t hi,
                           uint32_t need, uint32_t &T, uint32_t &rem,
                           bool &whole) const {
        // each pass shrinks the range by 2^LOG2NB; the bound only guards
        // against inconsistent counts
        for (int pass = 0; pass < 40; ++pass) {
            const uint32_t range = hi - lo;
            if (range == 0) {
                T = lo;
                rem = need;
                whole = false;
                return;
            }
            const int bw = bit_width(range);
            const int shift = bw > LOG2NB ? bw - LOG2NB : 0;
            clear_hist();
            G.sync();
            fe([&](uint32_t key, uint32_t pl) {
                bool v;
                uint32_t k;
                ext(key, pl, v, k);
                if (v && (k - lo) <= range) atomicAdd(&hist[(k - lo) >> shift], 1u);
            });
            G.sync();
            uint32_t b, above, cnt;
            crossing(need, b, above, cnt);
            need -= above;
            const uint32_t off = b << shift;
            const uint32_t nlo = lo + off;
            const uint32_t span = shift ? ((1u << shift) - 1u) : 0u;
            const uint32_t nhi = (range - off <= span) ? hi : nlo + span;
            if (cnt == need) {
                T = nlo;
                rem = 0;
                whole = true;
                return;
            }
            if (shift == 0) {
                T = nlo;
                rem = need;
                whole = false;
                return;
            }
            lo = nlo;
            hi = nhi;
        }
        T = lo;
        rem = need;
        whole = false;
    }

    // The rule selecting the m best of the n elements (1 <= m).
    template <class FE, class IDX>
    __device__ __forceinline__ Rule select(FE fe, IDX idx, uint32_t n, uint32_t m) const {
        if (m >= n) return Rule{0u, 0u};
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
        fe([&](uint32_t key, uint32_t) {
            mn = min(mn, key);
            mx = max(mx, key);
        });
        mn = G.reduce_min(mn);
        mx = G.reduce_max(mx);
        uint32_t T, rem;
        bool whole;
        narrow(fe, [](uint32_t key, uint32_t, bool &v, uint32_t &k) { v = true; k = key; },
               mn, mx, m, T, rem, whole);
        if (whole) return Rule{T, 0u};
        // equal keys at the boundary: the `rem` smallest indices win
        uint32_t mn2 = 0xFFFFFFFFu, mx2 = 0u;
        fe([&](uint32_t key, uint32_t pl) {
            if (key == T) {
                const uint32_t k2 = ~idx(pl);
                mn2 = min(mn2, k2);
                mx2 = max(mx2, k2);
            }
        });
        mn2 = G.reduce_min(mn2);
        mx2 = G.reduce_max(mx2);
        uint32_t T2, rem2;
        bool whole2;
        const uint32_t Tk = T;
        narrow(fe,
               [&](uint32_t key, uint32_t pl, bool &v, uint32_t &k) {
                   v = (key == Tk);
                   k = v ? ~idx(pl) : 0u;  // idx may be a memory read: only for ties
               },
               mn2, mx2, rem, T2, rem2, whole2);
        // indices are distinct, so the narrowing always ends whole (or on a
        // single element): take ~idx >= T2
        return Rule{T, T2};
    }

    // Bucket sort of the msel selected elements (fs(f) calls f(key,
    // payload) for each selected element the thread owns) by (key desc,
    // index asc); returns in registers, for t < MAXPER and
    // tid + t*NT < msel, one element's final position rpos[t], key rkey[t]
    // and payload rpl[t]. The group is synchronised on return, so bufk /
    // bufp (msel entries of LDS) may then be reused to stage the output.
    template <int MAXPER, class FS, class IDX, class PL>
    __device__ __forceinline__ void sort_ranks(FS fs, IDX idx, uint32_t msel, uint32_t *bufk,
                                               PL *bufp, uint32_t (&rpos)[MAXPER],
                                               uint32_t (&rkey)[MAXPER],
                                               uint32_t (&rpl)[MAXPER]) const {
        if (msel == 0) return;
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
        fs([&](uint32_t key, uint32_t) {
            mn = min(mn, key);
            mx = max(mx, key);
        });
        mn = G.reduce_min(mn);
        mx = G.reduce_max(mx);
        const uint32_t range = mx - mn;
        const int bw = bit_width(range);
        const int shift = bw > LOG2NB ? bw - LOG2NB : 0;
        clear_hist();
        G.sync();
        fs([&](uint32_t key, uint32_t) { atomicAdd(&hist[(mx - key) >> shift], 1u); });
        G.sync();
        {
            uint32_t loc = 0;
            for (int i = 0; i < BPT; ++i) loc += hist[G.tid * BPT + i];
            uint32_t run = G.excl_scan(loc);
            for (int i = 0; i < BPT; ++i) {
                uint32_t h = hist[G.tid * BPT + i];
                hist[G.tid * BPT + i] = run;
                run += h;
            }
        }
        G.sync();
        fs([&](uint32_t key, uint32_t pl) {
            uint32_t slot = atomicAdd(&hist[(mx - key) >> shift], 1u);
            if (slot < msel) {
                bufk[slot] = key;
                bufp[slot] = (PL)pl;
            }
        });
        G.sync();
#pragma unroll
        for (int t = 0; t < MAXPER; ++t) {
            const uint32_t s = G.tid + t * NT;
            if (s < msel) {
                const uint32_t key = bufk[s];
                const uint32_t pl = bufp[s];
                const uint32_t myidx = idx(pl);
                const uint32_t b = (mx - key) >> shift;
                const uint32_t end = min(hist[b], msel);
                const uint32_t beg = b ? hist[b - 1] : 0u;
                uint32_t rank = 0;
                for (uint32_t u = beg; u < end; ++u) {
                    const uint32_t k2 = bufk[u];
                    rank += (k2 > key) || (k2 == key && idx(bufp[u]) < myidx);
                }
                rpos[t] = beg + rank;
                rkey[t] = key;
                rpl[t] = pl;
            }
        }
        G.sync();
    }

    // Order the msel selected elements (fs(f) calls f(key, payload) for each
    // selected element the thread owns) by (key desc, index asc) through a
    // bucket sort: bufk/bufp (LDS, msel entries) receive the bucketed
    // elements; out(pos, key, payload) is then called once per element with
    // its final rank pos in [0, msel).
    template <class FS, class IDX, class PL, class OUT>
    __device__ __forceinline__ void sort_selected(FS fs, IDX idx, uint32_t msel, uint32_t *bufk,
                                  PL *bufp, OUT out) const {
        if (msel == 0) return;
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
        fs([&](uint32_t key, uint32_t) {
            mn = min(mn, key);
            mx = max(mx, key);
        });
        mn = G.reduce_min(mn);
        mx = G.reduce_max(mx);
        const uint32_t range = mx - mn;
        const int bw = bit_width(range);
        const int shift = bw > LOG2NB ? bw - LOG2NB : 0;
        clear_hist();
        G.sync();
        fs([&](uint32_t key, uint32_t) { atomicAdd(&hist[(mx - key) >> shift], 1u); });
        G.sync();
        // exclusive scan of the bucket counts, best bucket first
        {
            uint32_t loc = 0;
            for (int i = 0; i < BPT; ++i) loc += hist[G.tid * BPT + i];
            uint32_t run = G.excl_scan(loc);
            for (int i = 0; i < BPT; ++i) {
                uint32_t h = hist[G.tid * BPT + i];
                hist[G.tid * BPT + i] = run;
                run += h;
            }
        }
        G.sync();
        fs([&](uint32_t key, uint32_t pl) {
            uint32_t slot = atomicAdd(&hist[(mx - key) >> shift], 1u);
            if (slot < msel) {
                bufk[slot] = key;
                bufp[slot] = (PL)pl;
            }
        });
        G.sync();
        // hist[b] now ends bucket b; rank each element inside its bucket
        for (uint32_t s = G.tid; s < msel; s += NT) {
            const uint32_t key = bufk[s];
            const uint32_t pl = bufp[s];
            const uint32_t myidx = idx(pl);
            const uint32_t b = (mx - key) >> shift;
            const uint32_t end = min(hist[b], msel);
            const uint32_t beg = b ? hist[b - 1] : 0u;
            uint32_t rank = 0;
            for (uint32_t t = beg; t < end; ++t) {
                const uint32_t k2 = bufk[t];
                rank += (k2 > key) || (k2 == key && idx(bufp[t]) < myidx);
            }
            out(beg + rank, key, pl);
        }
        G.sync();
    }
};

}  // namespace pivot
