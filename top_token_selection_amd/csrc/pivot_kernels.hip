// pivot_kernels.hip -- HIP kernels of the PIVOT query-group indexer for
// CDNA4 (gfx950), and the C ABI that launches them (include/pivot.h).
//
// Method (arXiv abstract of "PIVOT: Efficient Query-Group Indexing for
// Token-Level Sparse Attention"; "PIVOT Explained", sections "How It Works"
// and "Show Me The Code"): a group of queries is averaged into a proxy; ONE
// causal prefix scan of the proxy against the keys gives a candidate set C
// of the K best keys; PIVOT-Refine re-scores C with each member query and
// keeps its own top_k, PIVOT-Reuse hands the proxy's top_k to the members.
//
// Pipeline of one prefill call (per chunk of heads):
//   k_proxy    q -> P (head-major (h, group, d)), float32 sum + IEEE divide
//   k_scan     (sample pass) proxy . every s-th key of the prefix, on bf16 /
//              fp32 MFMA; all sample scores kept
//   k_tau      per row: threshold tau = r-th best sample score, chosen so
//              that at least K keys of the full prefix score >= tau with
//              overwhelming probability
//   k_scan     (main pass) proxy . every key of the prefix on MFMA; only
//              scores >= tau leave the chip, as (key, index) survivors
//   k_select   per row: exact top-K of the survivors (Refine: candidate
//              list) or exact sorted top_k (Reuse / dense: output rows);
//              rows whose survivors cannot prove exactness are queued
//   k_fallback queued rows: recompute the whole prefix, exact selection
//   k_refine   per group: gather K[C], members' scores on MFMA, per-member
//              exact sorted top_k
// Decode replaces the scans by k_decode_scan (an HBM-streaming GEMV that
// writes every score of each (sequence, head) row); k_dec_tau takes the
// row's threshold from every s-th score, k_dec_filter streams the row once
// and keeps the scores >= tau as survivors, and the prefill selection
// (k_select_wave / k_select, queued rows through k_fallback) finishes it.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "../../include/pivot.h"
#include "pivot_device.hpp"

using namespace pivot;

// Scratch of pivot_index_decode_noalloc: device memory the library owns, one
// copy per GPU, held until the process ends. Host code never uses this name
// as an address (on the host it is a stand-in): it takes the device address
// from hipGetSymbolAddress, once per device.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)256 << 20;
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

constexpr int SCAN_THREADS = 512;  // 8 wavefronts
constexpr int SCAN_GB = 1;         // 32-group column blocks per wavefront
constexpr int SCAN_ROWS = SCAN_THREADS / 64 * 32 * SCAN_GB;  // groups per scan block
constexpr int SCAN_KEYS = 32;      // keys per k-tile
constexpr int RING = 16;           // staged survivors per (row, half) stream
constexpr int FLUSH = 8;           // survivors written per flush (64 bytes)
constexpr int SEL_THREADS = 256;
constexpr int SEL_LOG2NB = 11;
constexpr int SEL_E = 48;          // survivors per thread held in registers (Ksel <= 4096)
constexpr int SEL_E_BIG = 96;      // the same for Ksel up to MAX_K
constexpr int TAU_E = 16;          // samples per thread held in registers
constexpr int REF_LOG2NB = 10;
constexpr int REF_E = 64;          // candidates per lane (K <= REF_MAXK)
constexpr int REF_MAXK = 64 * REF_E;  // candidates one wavefront's registers hold
constexpr int REF_FIX = 48;        // staging entries per lane at most (top_k + slack <= 3072)
constexpr int REF_LOG2 = 11;       // fused select: 2048 buckets
constexpr int REF_NB = 1 << REF_LOG2;
constexpr int REF_LOG2C = 10;      // fused select: coarse bins
constexpr int REF_HDR = ((1 << REF_LOG2C) + 64 + REF_NB / 2 + 64 + 16) * 4;  // bytes before the staged entries
constexpr int MAX_K = 8192;
constexpr int MAX_TOPK = 8192;
constexpr int RS_E = MAX_K / SEL_THREADS;  // row select: candidate scores per thread
constexpr int SORT_MP = 16;        // sorted rows ranked in registers: up to SORT_MP * SEL_THREADS
constexpr int FB_BLOCKS = 256;
constexpr int DEC_THREADS = 256;
constexpr int DEC_TOKENS = 512;    // tokens per decode-scan block
constexpr int SW_E = 96;           // select (wave): positions per lane (6144 per row)
constexpr int SW_WAVES = 4;        // select (wave): rows per block
constexpr int SW_CAP = 2240;       // select (wave): staged entries per row
constexpr int SW_REG = REF_HDR + 4 * (SW_CAP + 64);  // select (wave): LDS bytes per row

// Hardware places block b on XCD b % 8; hand each XCD a contiguous range of
// logical work so neighbouring work shares that XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nb) {
    const uint32_t per = nb / 8u, rem = nb % 8u;
    const uint32_t x = b % 8u, i = b / 8u;
    return x * per + min(x, rem) + i;
}

// s_waitcnt on the LDS counter alone: wait until every LDS access of the
// wavefront is done (vmcnt and expcnt fields at their maxima: no wait on
// vector memory).
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

__device__ __forceinline__ int64_t prefix_len(int64_t j, int g) {
    const int64_t s = j * (int64_t)g;
    return s > 1 ? s : 1;
}

// virtual keys v = 0, 1, ... stand for keys koff + kstride * v; count of
// those below n
__device__ __forceinline__ int64_t virt_count(int64_t n, int kstride, int koff) {
    return n > koff ? (n - koff - 1) / kstride + 1 : 0;
}

// ------------------------------------------------------------------ proxy

template <typename T>
__global__ void k_proxy(const T *__restrict__ q, int64_t S, int H, int D, int g,
                        int h0, int Hc, int64_t G, int rep, T *__restrict__ P) {
    // each thread: V consecutive dims (16 bytes) of one proxy row, the
    // members read as 16-byte loads; per dimension the sum runs in position
    // order, as one element at a time would
    constexpr int V = 16 / (int)sizeof(T);
    const int DV = D / V;
    const int64_t total = (int64_t)Hc * G * DV;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int d0 = (int)(t % DV) * V;
        const int64_t row = t / DV;              // proxy row (hl, jr)
        const int64_t j = row % G / rep;         // rep proxy rows per group
        const int hl = (int)(row / G);
        const int64_t i0 = j * g;
        const int64_t m = min((int64_t)g, S - i0);
        const T *src = q + (i0 * H + (h0 + hl)) * (int64_t)D + d0;
        float sum[V];
#pragma unroll
        for (int v = 0; v < V; ++v) sum[v] = 0.f;
        for (int64_t i = 0; i < m; ++i) {
            const uint4 x = *(const uint4 *)(src + i * (int64_t)H * D);
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int v = 0; v < V; ++v) {
                float f;
                if constexpr (sizeof(T) == 4) f = __uint_as_float(w[v]);
                else f = __uint_as_float((v & 1) ? (w[v >> 1] & 0xFFFF0000u) : (w[v >> 1] << 16));
                sum[v] += f;
            }
        }
        T *dst = P + row * (int64_t)D + d0;
#pragma unroll
        for (int v = 0; v < V; ++v) store_from_f32(dst + v, __fdiv_rn(sum[v], (float)m));
    }
}

__global__ void k_zero_u32(uint32_t *p, int64_t n) {
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n;
         t += (int64_t)gridDim.x * blockDim.x)
        p[t] = 0u;
}

struct Offsets64 {
    int64_t v[64];
    int count;
    int start;
};
__global__ void k_put_offsets(int64_t *dst, Offsets64 a) {
    const int t = threadIdx.x;
    if (t < a.count) dst[a.start + t] = a.v[t];
}

// ------------------------------------------------------------------- scan

struct ScanParams {
    const void *P;
    int64_t p_row, p_head;  // element strides of a proxy row / local head
    const void *K;
    int64_t k_row;          // element stride between consecutive keys
    int64_t k_head0;        // element offset of the chunk's first head
    int64_t k_head;         // element stride between heads
    int64_t G;              // rows (groups) per head
    int g;                  // group size (prefix of row j = max(j*g, 1))
    int kstride, koff;      // key sampling
    const float *tau;       // per-row threshold, nullptr = keep all
    uint32_t *out;          // survivors [(row*2+half)*stride + slot]: (float bits, key) pairs,
                            // or float bits alone when score_only
    int score_only;         // write scores without keys (the sample pass)
    int cap_half;           // more than this many in a half = overflow
    int stride;             // slots per (row, half): cap_half + 32, a multiple of 8
    int *cnt;               // survivors per (row, half); > cap_half = overflow
    int64_t min_n;          // rows with prefix <= min_n are skipped
    int n_tiles, Hc;
};

// One block: SCAN_ROWS consecutive groups of one head against every key of
// their prefixes, 32 keys per step; each wavefront takes SCAN_GB column
// blocks of 32 groups. MFMA 32x32x16 with keys as the A operand (rows) and
// proxies as B (columns): lane l holds column l%32 of each 32x32 tile, i.e.
// one group, for 16 keys -- its threshold and running survivor count stay
// in registers. Two blocks share a CU (four wavefronts per SIMD).
//
// Key tiles are loaded into registers two steps ahead (the keys of a head
// are shared by the blocks of its groups, which are not in step: many loads
// miss the L2), then written to one of two LDS buffers with the 16-byte
// chunks of a key row XOR-swizzled by the row, so that the fragment reads
// spread over the banks. One step, for tile kt:
//   barrier                                 (tile kt is in LDS)
//   tile kt+1 from registers into LDS       (the buffer of tile kt-1)
//   issue the loads of tile kt+3            (into tile kt+1's registers)
//   matrix work on tile kt
//   filter tile kt-1's scores (survivor stores)
// so loads have two whole steps to complete before their wait, and stores
// are never waited for in the loop.
//
// Survivors ((float bits, key) pairs) of each (row, half) stream are staged
// in an LDS ring of RING entries and leave in whole 64-byte chunks of FLUSH
// entries, four lanes to a chunk, so that one store instruction writes up to
// 16 whole chunks of different streams. A stream that passes cap_half
// survivors stops keeping (its row takes the exact fallback).
template <typename T, int D, bool UNIT>
__global__ void __launch_bounds__(SCAN_THREADS, (sizeof(T) == 4 && D == 128) ? 2 : 4) k_scan(ScanParams p) {
    constexpr int GB = SCAN_GB;
    constexpr int RB = D * (int)sizeof(T);     // bytes per key row
    constexpr int NCK = RB / 16;               // 16-byte chunks per key row
    constexpr int SWZ = (NCK < 16 ? NCK : 16) - 1;
    constexpr int TILE = SCAN_KEYS * RB;       // bytes per LDS tile
    constexpr int PIECES = SCAN_KEYS * NCK;    // 16-byte pieces per tile
    constexpr int NLD = (PIECES + SCAN_THREADS - 1) / SCAN_THREADS;  // loads per thread per tile
    constexpr int NSTREAM = 2 * SCAN_ROWS;     // (row, half) streams per block
    static_assert(NSTREAM == GB * SCAN_THREADS, "one stream per lane and column block");
    extern __shared__ __align__(16) unsigned char smem[];
    // survivor rings (static LDS, so that addresses fold into offsets):
    // (score bits, key index) entries [RING][NSTREAM]; the key tiles are
    // the dynamic LDS
    __shared__ __align__(16) uint2 ringS[RING * NSTREAM];
    constexpr uint32_t RROW = NSTREAM * 8;         // bytes per ring row
    static_assert((RING & (RING - 1)) == 0 && (RROW & (RROW - 1)) == 0, "ring sizes are powers of two");
    static_assert(RROW == 0x1000, "the filter's count step is written as 0x1000");
    static_assert(FLUSH == 8, "a chunk is four lanes' 16-byte stores");

    // Heads go to XCDs in groups of ceil(Hc / 8) (each XCD's contiguous range
    // of logical blocks then covers about one group, whose blocks share the
    // keys in its L2), and inside a group the tiles run longest first across
    // all of its heads, so that no long tile starts late.
    const int nb = p.Hc * p.n_tiles;
    const uint32_t L = xcd_remap(blockIdx.x, (uint32_t)nb);
    const int hg = (p.Hc + 7) / 8;                      // heads per group
    const int grp = (int)(L / (uint32_t)(hg * p.n_tiles));
    const int in_grp = (int)(L % (uint32_t)(hg * p.n_tiles));
    const int hgc = min(hg, p.Hc - grp * hg);           // heads of this group
    const int hl = grp * hg + in_grp % hgc;
    const int tile = p.n_tiles - 1 - in_grp / hgc;      // longest first
    const int64_t j0 = (int64_t)tile * SCAN_ROWS;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int half = l >> 5;

    const int64_t jlast = min(j0 + SCAN_ROWS - 1, p.G - 1);
    const int64_t vmax = virt_count(prefix_len(jlast, p.g) > p.min_n ? prefix_len(jlast, p.g) : 0,
                                    p.kstride, p.koff);
    // keys below every row's count in this wavefront need no causal test
    // (rows past the last group keep nothing: the whole wavefront then
    // takes the causal test)
    int64_t vfull = 0;
    {
        const int64_t jw = j0 + 32 * GB * w;
        if (jw + 32 * GB - 1 < p.G && prefix_len(jw, p.g) > p.min_n)
            vfull = virt_count(prefix_len(jw, p.g), p.kstride, p.koff);
    }
    const float never = __builtin_nanf("");  // s >= NaN is false for every s

    // this lane's two streams: survivors kept so far (cs[gb]) and already
    // written (fl[gb]), both counted in units of RROW so that a count masked
    // to the ring is the ring row's byte offset; the stream's buffer sits at
    // byte offset soff0[gb] from the block's part of the survivor array.
    // pk[gb] describes the stream's next chunk for the flush: bits 13.. its
    // index in 64-byte units from the wavefront's part of the survivor
    // array, bits 0..12 the LDS byte offset / 8 of its first ring entry.
    unsigned char *sb = (unsigned char *)p.out + ((int64_t)hl * p.G + j0) * 2 * (int64_t)p.stride * 8;
    unsigned char *sbw = sb + (int64_t)(32 * GB * w) * 2 * (int64_t)p.stride * 8;
    // the same streams with 4-byte entries (score_only)
    unsigned char *sb4 = (unsigned char *)p.out + ((int64_t)hl * p.G + j0) * 2 * (int64_t)p.stride * 4;
    unsigned char *sbw4 = sb4 + (int64_t)(32 * GB * w) * 2 * (int64_t)p.stride * 4;
    const bool score_only = p.score_only != 0;
    uint32_t soff0[GB], cs[GB], fl[GB], pk[GB];
    int vcount[GB];
    float tau[GB];
    for (int gb = 0; gb < GB; ++gb) {
        cs[gb] = 0u;
        fl[gb] = 0u;
        const int jl = 32 * GB * w + 32 * gb + (l & 31);
        const int64_t j = j0 + jl;
        soff0[gb] = (uint32_t)((jl * 2 + half) * p.stride) * 8u;
        pk[gb] = ((uint32_t)(((32 * gb + (l & 31)) * 2 + half) * p.stride) / 8u << 13) |
                 (uint32_t)(gb * SCAN_THREADS + w * 64 + l);
        int64_t vc = 0;
        tau[gb] = never;  // rows past the end never keep
        if (j < p.G) {
            const int64_t n = prefix_len(j, p.g);
            if (n > p.min_n) vc = virt_count(n, p.kstride, p.koff);
            tau[gb] = p.tau ? p.tau[(int64_t)hl * p.G + j] : -INFINITY;
        }
        vcount[gb] = (int)vc;
    }
    const int stream0 = w * 64 + l;  // stream of gb is gb * SCAN_THREADS + stream0

    // proxies as resident B fragments
    typedef typename std::conditional<std::is_same<T, float>::value, f32x4_t, bf16x8_t>::type frag_t;
    constexpr int NKS = std::is_same<T, float>::value ? D / 8 : D / 16;
    frag_t bq[GB][NKS];
    const T *Pb = (const T *)p.P + (int64_t)hl * p.p_head;
    for (int gb = 0; gb < GB; ++gb) {
        const int64_t j = j0 + 32 * GB * w + 32 * gb + (l & 31);
        for (int ks = 0; ks < NKS; ++ks) {
            frag_t f;
            if (j < p.G) {
                const int dofs = std::is_same<T, float>::value ? 8 * ks + 4 * half : 16 * ks + 8 * half;
                f = *(const frag_t *)(Pb + j * p.p_row + dofs);
            } else {
                f = frag_t{};
            }
            bq[gb][ks] = f;
        }
    }

    const int ntiles_k = (int)((vmax + SCAN_KEYS - 1) / SCAN_KEYS);
    const unsigned char *Kb = (const unsigned char *)((const T *)p.K + p.k_head0 + (int64_t)hl * p.k_head);
    const int64_t krow_bytes = p.k_row * (int64_t)sizeof(T);
    // UNIT: every key (kstride 1), so that a score's key index is the tile's
    // plus a constant
    const uint32_t kstr = UNIT ? 1u : (uint32_t)p.kstride;
    const uint32_t lane_key = (uint32_t)p.koff + kstr * (uint32_t)(4 * half);

    // tile kt, staged through registers: piece i of a thread is 16-byte
    // chunk c = q % NCK of key row r = q / NCK of the tile, q = (4 i + w) 64
    // + l (consecutive lanes read consecutive chunks of a row), and goes to
    // LDS buffer kt & 1 at slot r NCK + (c ^ swz(r)): slot (r, pos) holds
    // chunk pos ^ swz(r). Keys past the last row's prefix repeat the last
    // key: their scores are never kept (that tile takes the causal test).
    typedef u32x4_t piece_t[NLD];
    // A tile's rows are read through a buffer resource whose base is the
    // tile's first key (scalar registers) and whose range ends after the
    // row of virtual key vmax - 1: this thread's piece sits at a fixed
    // offset from the base (below 2^32: the host refuses key strides that
    // would pass it), and rows past the range read as zero (their scores
    // are never kept).
    const uint32_t rstep = kstr * (uint32_t)krow_bytes;  // bytes between consecutive virtual keys
    const int64_t kend = vmax > 0 ? (p.koff + (int64_t)p.kstride * (vmax - 1)) * krow_bytes + RB : 0;
    uint32_t loff[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int q = min((i * (SCAN_THREADS / 64) + w) * 64 + l, PIECES - 1);
        loff[i] = (uint32_t)(q / NCK) * rstep + (uint32_t)(q % NCK) * 16u;
    }
    auto load_tile = [&](int kt, piece_t &pr) {
        const int64_t b0 = (p.koff + (int64_t)p.kstride * kt * SCAN_KEYS) * krow_bytes;
        const int64_t left = kend - b0;
        const uint32_t nrec = left <= 0 ? 0u : (left >= (int64_t)0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)left);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(Kb + b0), (short)0, (int)nrec, 0x00020000);
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            pr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)loff[i], 0, 0));
    };
    auto store_tile = [&](int kt, const piece_t &pr) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int q = (i * (SCAN_THREADS / 64) + w) * 64 + l;
            const int r = q / NCK, c = q % NCK;
            // threads past the tile's pieces (a tile smaller than one
            // piece per thread) store nothing
            if (PIECES % SCAN_THREADS == 0 || q < PIECES)
                *(u32x4_t *)(smem + (kt & 1) * TILE + (r * NCK + (c ^ (r & SWZ))) * 16) = pr[i];
        }
    };

    typedef f32x16_t acc_t[GB];
    // fragment of k-step ks: chunk (2 ks + half) ^ (r & SWZ) of tile row r,
    // i.e. LDS address A0 ^ (ks << 5) with A0 that of k-step 0 (the chunk
    // bits lie below the row's, and the tiles -- the dynamic LDS, which
    // starts right after the static rings -- are 512-byte aligned); A0 is
    // renewed opaquely every tile so that the eight addresses are formed in
    // the loop instead of held in registers
    static_assert((RING * NSTREAM * 8) % 512 == 0 && TILE % 512 == 0, "key tiles start 512-byte aligned");
    const uint32_t A0 = (uint32_t)(uintptr_t)smem + (uint32_t)((l & 31) * RB) +
                        ((uint32_t)(half ^ ((l & 31) & SWZ)) << 4);
    typedef __attribute__((address_space(3))) const unsigned char *lds_cptr;
    // All NKS fragments of a tile are read before its matrix work (the
    // scheduler would otherwise interleave one read and one MFMA at a time,
    // exposing the LDS latency eight times a step).
    auto matrix = [&](int kt, acc_t &acc) {
        uint32_t a0;
        asm volatile("" : "=v"(a0) : "0"(A0));
#pragma unroll
        for (int gb = 0; gb < GB; ++gb) acc[gb] = f32x16_t{};
        frag_t fa[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            fa[ks] = *(__attribute__((address_space(3))) const frag_t *)((lds_cptr)(uintptr_t)(a0 ^ (uint32_t)(ks << 5)) +
                                                                       (kt & 1) * TILE);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int gb = 0; gb < GB; ++gb) {
                if constexpr (std::is_same<T, float>::value) {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[gb] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[ks][v], bq[gb][ks][v], acc[gb], 0, 0, 0);
                } else {
                    acc[gb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks], bq[gb][ks], acc[gb], 0, 0, 0);
                }
            }
        }
    };

    // Every stream with FLUSH or more staged survivors sends its FLUSH
    // oldest (ring rows fl % RING ..) as one 64-byte chunk. The streams of
    // each column block are ranked; the r-th one passes pk (its chunk's
    // index and first ring entry) to lane 4r (forward permute, no LDS
    // memory) and over its quad (DPP), and lane 4r + q stores entries
    // 2q, 2q + 1 of the chunk (one LDS read of two ring rows): an
    // instruction writes 16 whole chunks. Both column blocks' passes run
    // side by side, so their LDS round trips overlap. At most cap_half + 16
    // are ever kept, inside the stream's stride. Wavefront-uniform control
    // flow.
    static_assert(RING == 2 * FLUSH, "a chunk starts at ring row 0 or FLUSH");
    static_assert(NSTREAM <= 1024, "ring entry offsets / 8 fit 13 bits");
    const uint32_t lds_q = 2u * (uint32_t)(l & 3) * RROW;  // ring rows 2q, 2q+1 of a chunk
    unsigned char *sbq = sbw + 16u * (uint32_t)(l & 3);    // entries 2q, 2q+1 of a chunk
    unsigned char *sbq4 = sbw4 + 8u * (uint32_t)(l & 3);   // the same, 4-byte entries
    auto flush = [&]() {
        bool need[GB];
        uint64_t M[GB];
        uint32_t rank[GB];
        int nf[GB];
        uint64_t any = 0;
        int nmax = 0;
#pragma unroll
        for (int gb = 0; gb < GB; ++gb) {
            need[gb] = cs[gb] - fl[gb] >= (uint32_t)FLUSH * RROW;
            M[gb] = __ballot(need[gb]);
            nf[gb] = __popcll(M[gb]);
            rank[gb] = __builtin_amdgcn_mbcnt_hi((uint32_t)(M[gb] >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)M[gb], 0u));
            any |= M[gb];
            nmax = max(nmax, nf[gb]);
        }
        if (any == 0) return;
        for (int r0 = 0; r0 < nmax; r0 += 16) {
            uint32_t got[GB];
#pragma unroll
            for (int gb = 0; gb < GB; ++gb) {
                // senders target lane 4 (rank - r0); the others an odd lane
                const bool mine = need[gb] && rank[gb] - (uint32_t)r0 < 16u;
                const int to = mine ? (int)(rank[gb] - (uint32_t)r0) * 16 : (l | 1) * 4;
                got[gb] = dpp_u32<0x00>(0u, (uint32_t)__builtin_amdgcn_ds_permute(to, (int)pk[gb]));
            }
#pragma unroll
            for (int gb = 0; gb < GB; ++gb) {
                if ((l >> 2) < nf[gb] - r0) {
                    const uint2 *e = (const uint2 *)((unsigned char *)ringS + (((got[gb] & 0x1FFFu) << 3) | lds_q));
                    const uint2 a = e[0], b = e[NSTREAM];
                    if (score_only) *(uint2 *)(sbq4 + (got[gb] >> 13) * 32u) = make_uint2(a.x, b.x);
                    else *(uint4 *)(sbq + (got[gb] >> 13) * 64u) = make_uint4(a.x, a.y, b.x, b.y);
                }
            }
        }
#pragma unroll
        for (int gb = 0; gb < GB; ++gb) {
            // next chunk: one further in the array, the other half of the ring
            fl[gb] += need[gb] ? (uint32_t)FLUSH * RROW : 0u;
            pk[gb] = need[gb] ? (pk[gb] + (1u << 13)) ^ (FLUSH * RROW / 8u) : pk[gb];
        }
    };

    // keep the scores of tile kt that reach the row's threshold; at most 16
    // per stream and tile. Tiles below every row's prefix end skip the causal
    // test. Flushes keep the ring from filling: at a step's end every stream
    // with 8 or more waiting sends one chunk, so at most 8 wait when a step
    // starts; after its first 8 scores (at most 16 waiting) the flush runs
    // only if some stream has more than 8 waiting, so that its next 8 fit.
    // Per score: one compare (two on causal tiles), the ring slot address
    // from the count (one and-or) and the key index; then, with exec set to
    // the lanes that keep the score (their ballot) and restored at once, one
    // LDS instruction stores score bits and key index from their own
    // registers and one add steps the count: no branch, and the other lanes
    // neither write nor count.
    auto filter = [&](int kt, const acc_t &acc) {
#pragma unroll
        for (int gb = 0; gb < GB; ++gb)
            if (cs[gb] > (uint32_t)p.cap_half * RROW) tau[gb] = never;
        const uint32_t tkey = kstr * (uint32_t)(kt * SCAN_KEYS) + lane_key;
        auto run = [&](auto causal) {
#pragma unroll
            for (int hv = 0; hv < 2; ++hv) {
#pragma unroll
                for (int gb = 0; gb < GB; ++gb) {
                    // byte offset of this stream's column in a ring row
                    const uint32_t col = (uint32_t)(gb * SCAN_THREADS + stream0) * 8u;
                    // rows' key bound relative to this lane's first key of the tile
                    const int lim = vcount[gb] - (kt * SCAN_KEYS + 4 * half);
#pragma unroll
                    for (int v = 8 * hv; v < 8 * hv + 8; ++v) {
                        const int vo = 8 * (v >> 2) + (v & 3);
                        const float sc = acc[gb][v];
                        bool keep = sc >= tau[gb];
                        if constexpr (decltype(causal)::value) keep = keep && (vo < lim);
                        // only the lanes that keep write (exec = their ballot,
                        // restored at once: no branch); they also count
                        const uint32_t slot = (uint32_t)(uintptr_t)ringS + ((cs[gb] & ((RING - 1) * RROW)) | col);
                        const uint64_t km = __builtin_amdgcn_ballot_w64(keep);
                        uint64_t sv;
                        asm volatile(
                            "s_and_saveexec_b64 %[sv], %[km]\n\t"
                            "ds_write2_b32 %[a], %[x], %[y] offset1:1\n\t"
                            "v_add_u32_e32 %[c], 0x1000, %[c]\n\t"
                            "s_mov_b64 exec, %[sv]"
                            : [sv] "=&s"(sv), [c] "+v"(cs[gb])
                            : [km] "s"(km), [a] "v"(slot), [x] "v"(__float_as_uint(sc)),
                              [y] "v"(tkey + kstr * (uint32_t)vo)
                            : "memory");
                    }
                }
                if (hv == 1) {
                    flush();
                } else {
                    // at most 8 wait at a step's start: the mid-step flush is
                    // needed only where more than 8 wait now
                    bool over = false;
#pragma unroll
                    for (int gb = 0; gb < GB; ++gb) over = over || (cs[gb] - fl[gb] > (uint32_t)FLUSH * RROW);
                    if (__builtin_amdgcn_ballot_w64(over) != 0) flush();
                }
            }
        };
        if ((int64_t)(kt + 1) * SCAN_KEYS <= vfull) run(std::false_type{});
        else run(std::true_type{});
    };

    // Four tiles are in flight in registers while one is in LDS. Step kt:
    // the barrier (after this wavefront's LDS writes are done) makes tile
    // kt, written by every wavefront in the previous step, readable, and
    // frees the buffer of tile kt-1; tile kt+1 (loaded four steps ago) goes
    // there, and its registers take the loads of tile kt+5; then tile kt's
    // scores are computed and filtered. The compiler's wait before the LDS
    // writes counts the three later tile loads, so survivor stores of the
    // last steps need not have completed.
    auto step = [&](int kt, acc_t &acc, piece_t &nxt) {
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        // unconditional (tiles past the last read zeros), so that the
        // compiler's count of loads in flight is exact
        store_tile(kt + 1, nxt);
        load_tile(kt + 5, nxt);
        matrix(kt, acc);
        filter(kt, acc);
    };
    // every proxy fragment has arrived before the loop. Tile t stages in
    // P[t % 4] (four steps per iteration keep the names static).
    __builtin_amdgcn_s_waitcnt(0);
    {
        acc_t acc;
        piece_t P0, P1, P2, P3;
        if (ntiles_k > 0) {
            load_tile(0, P0);
            load_tile(1, P1);
            load_tile(2, P2);
            load_tile(3, P3);
            store_tile(0, P0);
            load_tile(4, P0);
        }
        int kt = 0;
        for (; kt + 4 <= ntiles_k; kt += 4) {
            step(kt, acc, P1);
            step(kt + 1, acc, P2);
            step(kt + 2, acc, P3);
            step(kt + 3, acc, P0);
        }
        if (kt < ntiles_k) step(kt, acc, P1);
        if (kt + 1 < ntiles_k) step(kt + 1, acc, P2);
        if (kt + 2 < ntiles_k) step(kt + 2, acc, P3);
    }

    // the rest of each ring (fewer than FLUSH entries) one by one
    for (int gb = 0; gb < GB; ++gb) {
        const uint2 *rs = ringS + gb * SCAN_THREADS + stream0;
        const uint32_t cnt = cs[gb] / RROW;
        for (uint32_t e = fl[gb] / RROW; e < cnt; ++e) {
            if (score_only) *(uint32_t *)(sb4 + soff0[gb] / 2u + e * 4u) = rs[(e % RING) * NSTREAM].x;
            else *(uint2 *)(sb + soff0[gb] + e * 8u) = rs[(e % RING) * NSTREAM];
        }
        const int64_t j = j0 + 32 * GB * w + 32 * gb + (l & 31);
        if (j < p.G) p.cnt[((int64_t)hl * p.G + j) * 2 + half] = (int)cnt;
    }
}

// -------------------------------------------------------------------- tau

struct TauParams {
    const uint32_t *samp;   // samples: float bits
    const int *scnt;
    int samp_half, samp_stride;
    float *tau;
    int64_t G;
    int g;
    int64_t keep_all_n;  // rows with prefix <= this keep every key
    int64_t rsel;        // rank of the threshold sample
};

// Per row: tau = the rsel-th best sample score (-inf when the row keeps
// every key or has too few samples -- then k_select finds the overflow and
// the row takes the exact fallback). Register slots past the samples hold
// key 0, which no finite score maps to, so they never rank.
__global__ void __launch_bounds__(SEL_THREADS) k_tau(TauParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *hist = (uint32_t *)smem;
    uint32_t *vars = hist + (1 << SEL_LOG2NB);
    uint32_t *red = vars + 8;
    const int64_t r = blockIdx.x;
    const int64_t j = r % p.G;
    const int64_t n = prefix_len(j, p.g);
    if (n <= p.keep_all_n) {
        if (threadIdx.x == 0) p.tau[r] = -INFINITY;
        return;
    }
    const int c0 = min(p.scnt[2 * r], p.samp_half), c1 = min(p.scnt[2 * r + 1], p.samp_half);
    const uint32_t ns = min((uint32_t)(c0 + c1), (uint32_t)(TAU_E * SEL_THREADS));
    if ((int64_t)ns <= p.rsel) {
        if (threadIdx.x == 0) p.tau[r] = -INFINITY;
        return;
    }
    Group<4> G{(int)threadIdx.x, red};
    Selector<4, SEL_LOG2NB> sel{G, hist, vars};
    const int elim = (int)((ns + SEL_THREADS - 1) / SEL_THREADS);
    uint32_t key[TAU_E];
    const uint32_t *b0 = p.samp + (2 * r) * (int64_t)p.samp_stride;
    const uint32_t *b1 = p.samp + (2 * r + 1) * (int64_t)p.samp_stride;
    bool has[TAU_E];
#pragma unroll
    for (int e = 0; e < TAU_E; ++e) {
        const uint32_t gi = e * SEL_THREADS + threadIdx.x;
        has[e] = e < elim && gi < ns;
        key[e] = has[e] ? (gi < (uint32_t)c0 ? b0[gi] : b1[gi - c0]) : 0u;
    }
#pragma unroll
    for (int e = 0; e < TAU_E; ++e) key[e] = has[e] ? score_key(__uint_as_float(key[e])) : 0u;
    auto fe = [&](auto f) {
#pragma unroll
        for (int e = 0; e < TAU_E; ++e)
            if (e < elim) f(key[e], e * SEL_THREADS + threadIdx.x);
    };
    const Rule rule = sel.select(fe, [](uint32_t x) { return x; }, (uint32_t)elim * SEL_THREADS,
                                 (uint32_t)p.rsel);
    if (threadIdx.x == 0) p.tau[r] = key_score(rule.T);
}

// ----------------------------------------------------------------- select

struct RowOut {
    // candidate mode (Refine): list of K' indices per row
    uint32_t *cand;
    int64_t K;
    // output mode (Reuse / dense): sorted rows written for every member
    int32_t *out_idx;
    float *out_score;
    int top_k;
    int H, h0;
    int64_t S;
    int g;
};

// Writes the selected, ordered entry `pos` of group (hl, j) to every member
// row of the group (prefill layout).
__device__ __forceinline__ void put_member_rows(const RowOut &o, int hl, int64_t j, uint32_t pos,
                                                uint32_t key, uint32_t idx) {
    const int64_t i0 = j * o.g;
    const int64_t m = min((int64_t)o.g, o.S - i0);
    for (int64_t t = 0; t < m; ++t) {
        const int64_t off = ((i0 + t) * o.H + o.h0 + hl) * (int64_t)o.top_k + pos;
        o.out_idx[off] = (int32_t)idx;
        if (o.out_score) o.out_score[off] = key_score(key);
    }
}

__device__ void pad_member_rows(const RowOut &o, int hl, int64_t j, uint32_t from, int tid, int nt) {
    const int64_t i0 = j * o.g;
    const int64_t m = min((int64_t)o.g, o.S - i0);
    for (int64_t t = 0; t < m; ++t) {
        const int64_t base = ((i0 + t) * o.H + o.h0 + hl) * (int64_t)o.top_k;
        for (uint32_t pos = from + tid; pos < (uint32_t)o.top_k; pos += nt) {
            o.out_idx[base + pos] = -1;
            if (o.out_score) o.out_score[base + pos] = -INFINITY;
        }
    }
}

struct SelParams {
    const uint2 *surv;
    const int *cnt;
    int cap_half, stride;
    int64_t G;
    int g;
    int64_t Ksel;     // how many to select (K for Refine, top_k otherwise)
    int sorted_out;   // 0: candidate list, 1: sorted member rows
    RowOut o;
    uint32_t *fb_list;
    uint32_t *fb_count;
    // sorted rows: k_select_wave lists here the rows it leaves to k_select,
    // which then walks the list (list != 0) instead of one row per block
    uint32_t *big_list;
    uint32_t *big_count;
    int64_t rows;
    int list;
    // decode: B+1 prefix offsets of the sequences (row length of sequence j
    // is offs[j+1] - offs[j]); null in prefill (causal prefix of group j)
    const int64_t *offs;
    int buf_cap;      // entries of each LDS sort buffer (>= Ksel)
};

__device__ __forceinline__ int64_t sel_row_len(const SelParams &p, int64_t j) {
    return p.offs ? p.offs[j + 1] - p.offs[j] : prefix_len(j, p.g);
}

// Copies a staged row (LDS, msel valid entries) into every member row of
// group (hl, j), -1 / -inf past msel; coalesced stores.
__device__ __forceinline__ void write_member_rows(const RowOut &o, int hl, int64_t j,
                                                  const uint32_t *stage, uint32_t msel,
                                                  bool scores) {
    const int64_t i0 = j * o.g;
    const int64_t m = min((int64_t)o.g, o.S - i0);
    for (int64_t t = 0; t < m; ++t) {
        const int64_t base = ((i0 + t) * o.H + o.h0 + hl) * (int64_t)o.top_k;
        for (uint32_t c = threadIdx.x; c < (uint32_t)o.top_k; c += SEL_THREADS) {
            if (scores) o.out_score[base + c] = c < msel ? key_score(stage[c]) : -INFINITY;
            else o.out_idx[base + c] = c < msel ? (int32_t)stage[c] : -1;
        }
    }
}

// One block per row: the survivors of the main scan (a superset of the
// row's best Ksel keys when the row is not queued) are held in registers and
// the exact best min(Ksel, n) of them selected. Slots past the survivors
// hold key 0 (below every score) and never rank.
template <bool SORTED, int E>
__device__ __forceinline__ void select_row(const SelParams &p, const int64_t r, unsigned char *smem) {
    uint32_t *hist = (uint32_t *)smem;
    uint32_t *vars = hist + (1 << SEL_LOG2NB);
    uint32_t *red = vars + 8;
    uint32_t *ctr = red + 16;
    uint32_t *bufk = ctr + 4;
    uint32_t *bufp = bufk + p.buf_cap;

    const int64_t j = r % p.G;
    const int hl = (int)(r / p.G);
    const int64_t n = sel_row_len(p, j);
    const int c0 = p.cnt[2 * r], c1 = p.cnt[2 * r + 1];
    const uint32_t msel = (uint32_t)min(p.Ksel, n);
    if (c0 > p.cap_half || c1 > p.cap_half || (uint32_t)(c0 + c1) < msel) {
        if (threadIdx.x == 0) {
            const uint32_t slot = atomicAdd(p.fb_count, 1u);
            p.fb_list[slot] = (uint32_t)r;
        }
        return;
    }
    const uint32_t ns = (uint32_t)(c0 + c1);
    const int elim = (int)((ns + SEL_THREADS - 1) / SEL_THREADS);
    Group<4> G{(int)threadIdx.x, red};
    Selector<4, SEL_LOG2NB> sel{G, hist, vars};
    const uint2 *b0 = p.surv + (2 * r) * (int64_t)p.stride;
    const uint2 *b1 = p.surv + (2 * r + 1) * (int64_t)p.stride;
    auto ident = [](uint32_t x) { return x; };
    if constexpr (!SORTED) {
        uint32_t key[E], pl[E];
        // all loads first (independent, in flight together), then the keys
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t gi = e * SEL_THREADS + threadIdx.x;
            uint2 x = make_uint2(0u, 0xFFFFFFFFu);
            if (e < elim && gi < ns) x = gi < (uint32_t)c0 ? b0[gi] : b1[gi - c0];
            key[e] = x.x;
            pl[e] = x.y;
        }
#pragma unroll
        for (int e = 0; e < E; ++e)
            key[e] = pl[e] == 0xFFFFFFFFu ? 0u : score_key(__uint_as_float(key[e]));
        auto fe = [&](auto f) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (e < elim) f(key[e], pl[e]);
        };
        const Rule rule = msel >= ns ? Rule{0u, 0u}
                                     : sel.select(fe, ident, (uint32_t)elim * SEL_THREADS, msel);
        if (threadIdx.x == 0) ctr[0] = 0;
        __syncthreads();
        uint32_t *dst = p.o.cand + r * p.o.K;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (e < elim && key[e] != 0u && rule.sel(key[e], pl[e])) {
                const uint32_t slot = atomicAdd(&ctr[0], 1u);
                if (slot < msel) dst[slot] = pl[e];
            }
    } else {
        uint32_t key[E], pl[E];
        // all loads first (independent, in flight together), then the keys
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t gi = e * SEL_THREADS + threadIdx.x;
            uint2 x = make_uint2(0u, 0xFFFFFFFFu);
            if (e < elim && gi < ns) x = gi < (uint32_t)c0 ? b0[gi] : b1[gi - c0];
            key[e] = x.x;
            pl[e] = x.y;
        }
#pragma unroll
        for (int e = 0; e < E; ++e)
            key[e] = pl[e] == 0xFFFFFFFFu ? 0u : score_key(__uint_as_float(key[e]));
        auto fe = [&](auto f) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (e < elim) f(key[e], pl[e]);
        };
        const Rule rule = msel >= ns ? Rule{0u, 0u}
                                     : sel.select(fe, ident, (uint32_t)elim * SEL_THREADS, msel);
        auto fs = [&](auto f) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (e < elim && key[e] != 0u && rule.sel(key[e], pl[e])) f(key[e], pl[e]);
        };
        if constexpr (E > SEL_E) {
            if (msel > (uint32_t)(SORT_MP * SEL_THREADS)) {
                // more than the registers rank: every entry straight to its
                // member rows
                sel.sort_selected(fs, ident, msel, bufk, bufp, [&](uint32_t pos, uint32_t k, uint32_t idx) {
                    put_member_rows(p.o, hl, j, pos, k, idx);
                });
                pad_member_rows(p.o, hl, j, msel, (int)threadIdx.x, SEL_THREADS);
                return;
            }
        }
        uint32_t rpos[SORT_MP], rkey[SORT_MP], rpl[SORT_MP];
        sel.template sort_ranks<SORT_MP>(fs, ident, msel, bufk, bufp, rpos, rkey, rpl);
#pragma unroll
        for (int t = 0; t < SORT_MP; ++t)
            if (threadIdx.x + t * SEL_THREADS < msel) bufk[rpos[t]] = rpl[t];
        __syncthreads();
        write_member_rows(p.o, hl, j, bufk, msel, false);
        if (p.o.out_score) {
            __syncthreads();
#pragma unroll
            for (int t = 0; t < SORT_MP; ++t)
                if (threadIdx.x + t * SEL_THREADS < msel) bufk[rpos[t]] = rkey[t];
            __syncthreads();
            write_member_rows(p.o, hl, j, bufk, msel, true);
        }
    }
}

// SORTED: sorted member rows (Reuse, dense); otherwise candidate lists
// (Refine), which need fewer registers: three blocks share a CU. E: survivors
// per thread (SEL_E_BIG for Ksel above 4096, one block per CU).
template <bool SORTED, int E>
__global__ void __launch_bounds__(SEL_THREADS, E > SEL_E ? 1 : (SORTED ? 2 : 3)) k_select(SelParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    if (!p.list) {
        select_row<SORTED, E>(p, blockIdx.x, smem);
        return;
    }
    const uint32_t nl = *p.big_count;
    for (uint32_t it = blockIdx.x; it < nl; it += gridDim.x) {
        select_row<SORTED, E>(p, (int64_t)p.big_list[it], smem);
        __syncthreads();
    }
}

// --------------------------------------------------------------- fallback

struct FbParams {
    // prefill: rows come from the queue and are rescored here
    const uint32_t *fb_list;
    const uint32_t *fb_count;
    const void *P;
    int64_t p_row, p_head;
    const void *K;
    int64_t k_row, k_head0, k_head;
    int64_t G;
    int g;
    uint32_t *scratch;  // FB_BLOCKS rows of n_max keys
    int64_t n_max;
    // decode: queued rows r = head * B + sequence, scores already in `dense`
    int decode;
    const uint32_t *dense;
    const int64_t *offs;  // B+1 prefix offsets of the sequences
    int B, H;
    int64_t Ksel;
    int sorted_out;
    RowOut o;
    int D;
    int buf_cap;  // entries of each LDS sort buffer (>= Ksel)
};

// Streaming exact selection over a whole score row in global memory (the
// row is re-read once per narrowing pass).
template <typename T>
__global__ void __launch_bounds__(SEL_THREADS) k_fallback(FbParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *hist = (uint32_t *)smem;
    uint32_t *vars = hist + (1 << SEL_LOG2NB);
    uint32_t *red = vars + 8;
    uint32_t *ctr = red + 16;
    uint32_t *bufk = ctr + 4;
    uint32_t *bufp = bufk + p.buf_cap;
    float *prow = (float *)(bufp + p.buf_cap);  // D floats

    Group<4> G{(int)threadIdx.x, red};
    Selector<4, SEL_LOG2NB> sel{G, hist, vars};
    const int tid = threadIdx.x;
    const uint32_t nrows = *p.fb_count;

    for (uint32_t it = blockIdx.x; it < nrows; it += gridDim.x) {
        const uint32_t *keys;
        int64_t n;
        int hl;
        int64_t j;
        if (!p.decode) {
            const int64_t r = p.fb_list[it];
            j = r % p.G;
            hl = (int)(r / p.G);
            n = prefix_len(j, p.g);
            const T *pr = (const T *)p.P + hl * p.p_head + j * p.p_row;
            for (int d = tid; d < p.D; d += SEL_THREADS) prow[d] = load_f32(pr + d);
            __syncthreads();
            uint32_t *dst = p.scratch + (int64_t)blockIdx.x * p.n_max;
            const T *Kb = (const T *)p.K + p.k_head0 + (int64_t)hl * p.k_head;
            for (int64_t c = tid; c < n; c += SEL_THREADS) {
                const T *kr = Kb + c * p.k_row;
                float acc = 0.f;
                for (int d = 0; d < p.D; ++d) acc = fmaf(prow[d], load_f32(kr + d), acc);
                dst[c] = score_key(acc);
            }
            __syncthreads();
            keys = dst;
        } else {
            const uint32_t r = p.fb_list[it];
            const int b = (int)(r % (uint32_t)p.B);
            hl = (int)(r / (uint32_t)p.B);
            j = b;
            const int64_t off = p.offs[b];
            n = p.offs[b + 1] - off;
            keys = p.dense + off * p.H + (int64_t)hl * n;
        }
        const uint32_t msel = (uint32_t)min(p.Ksel, n);
        auto fe = [&](auto f) {
            for (int64_t c = tid; c < n; c += SEL_THREADS) f(keys[c], (uint32_t)c);
        };
        auto ident = [](uint32_t x) { return x; };
        const Rule rule = sel.select(fe, ident, (uint32_t)n, msel);
        auto fs = [&](auto f) {
            for (int64_t c = tid; c < n; c += SEL_THREADS) {
                const uint32_t k = keys[c];
                if (rule.sel(k, (uint32_t)c)) f(k, (uint32_t)c);
            }
        };
        const int64_t row = (int64_t)hl * (p.decode ? p.B : p.G) + j;
        if (!p.sorted_out) {
            if (tid == 0) ctr[0] = 0;
            __syncthreads();
            uint32_t *dst = p.o.cand + row * p.o.K;
            fs([&](uint32_t, uint32_t idx) {
                const uint32_t slot = atomicAdd(&ctr[0], 1u);
                if (slot < msel) dst[slot] = idx;
            });
        } else if (!p.decode) {
            sel.sort_selected(fs, ident, msel, bufk, bufp,
                              [&](uint32_t pos, uint32_t k, uint32_t idx) {
                                  put_member_rows(p.o, hl, j, pos, k, idx);
                              });
            pad_member_rows(p.o, hl, j, msel, tid, SEL_THREADS);
        } else {
            // decode member rows: b*g .. b*g+g-1
            const RowOut &o = p.o;
            sel.sort_selected(fs, ident, msel, bufk, bufp,
                              [&](uint32_t pos, uint32_t k, uint32_t idx) {
                                  for (int t = 0; t < o.g; ++t) {
                                      const int64_t off =
                                          (((int64_t)j * o.g + t) * o.H + hl) * (int64_t)o.top_k + pos;
                                      o.out_idx[off] = (int32_t)idx;
                                      if (o.out_score) o.out_score[off] = key_score(k);
                                  }
                              });
            for (int t = 0; t < o.g; ++t) {
                const int64_t base = (((int64_t)j * o.g + t) * o.H + hl) * (int64_t)o.top_k;
                for (uint32_t pos = msel + tid; pos < (uint32_t)o.top_k; pos += SEL_THREADS) {
                    o.out_idx[base + pos] = -1;
                    if (o.out_score) o.out_score[base + pos] = -INFINITY;
                }
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ decode scan

struct DecScanParams {
    const void *P;   // (H, B, D) proxies
    const void *kc;  // (sum ctx, H, D)
    const int64_t *offs;
    int B, H;
    int64_t max_chunks;
    uint32_t *dense;  // row (b, h) at offs[b]*H + h*ctx_b
};

// Streams the key cache once. Block = (sequence, group of 4 heads,
// DEC_TOKENS-token chunk), 4 wavefronts. A load instruction of a wavefront
// reads the 4 heads' key rows of one token (contiguous in the cache): 16
// lanes per row, lane j reading the j-th sixteenth of the row (its slice of
// its head's proxy stays in registers); the 16 partial dot products of a row
// are summed with DPP row shifts, lane 15 of the row ending with the score.
template <typename T, int D>
__global__ void __launch_bounds__(DEC_THREADS) k_decode_scan(DecScanParams p) {
    constexpr int RB = D * (int)sizeof(T);  // bytes per key row
    constexpr int CH = RB / 16;             // bytes per lane per row (8, 16 or 32)
    constexpr int NE = CH / (int)sizeof(T); // elements per lane per row
    constexpr int U = 32;                   // tokens per wavefront in flight
    typedef typename std::conditional<CH == 8, uint2, uint4>::type chunk_t;
    constexpr int NCH = CH >= 16 ? CH / 16 : 1;  // chunk_t loads per row
    const int ngrp = (p.H + 3) / 4;
    const int64_t per_seq = (int64_t)ngrp * p.max_chunks;
    const int b = (int)(blockIdx.x / per_seq);
    const int hg = (int)((blockIdx.x % per_seq) / p.max_chunks);
    const int64_t chunk = blockIdx.x % p.max_chunks;
    const int64_t off = p.offs[b];
    const int64_t ctx = p.offs[b + 1] - off;
    const int64_t t0 = chunk * DEC_TOKENS;
    if (t0 >= ctx) return;
    const int64_t t1 = min(t0 + (int64_t)DEC_TOKENS, ctx);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, j = l & 15, rr = l >> 4;
    const int h = min(4 * hg + rr, p.H - 1);  // lanes past the last head repeat it
    const bool live = 4 * hg + rr < p.H;

    float pv[NE];
    {
        const T *P = (const T *)p.P + ((int64_t)h * p.B + b) * D + NE * j;
#pragma unroll
        for (int e = 0; e < NE; ++e) pv[e] = load_f32(P + e);
    }
    const unsigned char *base = (const unsigned char *)((const T *)p.kc + (off * p.H + h) * (int64_t)D) + CH * j;
    const int64_t tstride = (int64_t)p.H * RB;  // bytes between consecutive tokens
    uint32_t *out = p.dense + off * p.H + (int64_t)h * ctx;

    // wavefront w takes tokens tb + w + 4u (u < U) of each block step
    for (int64_t tb = t0; tb < t1; tb += 4 * U) {
        chunk_t raw[U][NCH];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = min(tb + w + 4 * u, t1 - 1);
            const chunk_t *src = (const chunk_t *)(base + t * tstride);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                // streamed once: nontemporal, so the cache keeps the scores
                // the selection reads next
                if constexpr (sizeof(chunk_t) == 16) {
                    const u32x4_t x = __builtin_nontemporal_load((const u32x4_t *)(src + c));
                    raw[u][c] = make_uint4(x[0], x[1], x[2], x[3]);
                } else {
                    const u32x2_t x = __builtin_nontemporal_load((const u32x2_t *)(src + c));
                    raw[u][c] = make_uint2(x[0], x[1]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float acc = 0.f;
            if constexpr (std::is_same<T, float>::value) {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    acc = fmaf(pv[4 * c + 0], __uint_as_float(raw[u][c].x), acc);
                    acc = fmaf(pv[4 * c + 1], __uint_as_float(raw[u][c].y), acc);
                    acc = fmaf(pv[4 * c + 2], __uint_as_float(raw[u][c].z), acc);
                    acc = fmaf(pv[4 * c + 3], __uint_as_float(raw[u][c].w), acc);
                }
            } else if constexpr (CH == 8) {
                const uint32_t wds[2] = {raw[u][0].x, raw[u][0].y};
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2) {
                    acc = fmaf(pv[2 * q2], __uint_as_float(wds[q2] << 16), acc);
                    acc = fmaf(pv[2 * q2 + 1], __uint_as_float(wds[q2] & 0xFFFF0000u), acc);
                }
            } else {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const uint32_t wds[4] = {raw[u][c].x, raw[u][c].y, raw[u][c].z, raw[u][c].w};
#pragma unroll
                    for (int q2 = 0; q2 < 4; ++q2) {
                        acc = fmaf(pv[8 * c + 2 * q2], __uint_as_float(wds[q2] << 16), acc);
                        acc = fmaf(pv[8 * c + 2 * q2 + 1], __uint_as_float(wds[q2] & 0xFFFF0000u), acc);
                    }
                }
            }
            // sum over the 16 lanes of the row: lane 15 of the row gets it
            uint32_t x = __float_as_uint(acc);
            auto fadd = [](uint32_t a2, uint32_t b2) { return __float_as_uint(__uint_as_float(a2) + __uint_as_float(b2)); };
            x = fadd(x, dpp_u32<DPP_ROW_SHR1>(0u, x));
            x = fadd(x, dpp_u32<DPP_ROW_SHR2>(0u, x));
            x = fadd(x, dpp_u32<DPP_ROW_SHR4>(0u, x));
            x = fadd(x, dpp_u32<DPP_ROW_SHR8>(0u, x));
            const int64_t t = tb + w + 4 * u;
            if (j == 15 && live && t < t1) out[t] = score_key(__uint_as_float(x));
        }
    }
}

// ---------------------------------------------------- decode thresholds

struct DecTauParams {
    const uint32_t *dense;  // score keys of k_decode_scan
    int sshift;             // samples: keys 2^sshift - 1, 2 * 2^sshift - 1, ...
    const int64_t *offs;
    int B, H;
    int64_t keep_all_n, rsel;
    uint32_t *tau_key;  // per row h * B + b: keys >= it survive
};

// Per (sequence, head) row: the threshold key is the rsel-th best of the
// row's samples, every 2^sshift-th key (key 0 -- every key survives -- when
// the row keeps all its keys or has too few samples; the selection then
// finds the overflow and queues the row for the exact fallback).
__global__ void __launch_bounds__(SEL_THREADS) k_dec_tau(DecTauParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *hist = (uint32_t *)smem;
    uint32_t *vars = hist + (1 << SEL_LOG2NB);
    uint32_t *red = vars + 8;
    const int64_t r = blockIdx.x;
    const int b = (int)(r % p.B);
    const int hl = (int)(r / p.B);
    const int64_t off = p.offs[b];
    const int64_t n = p.offs[b + 1] - off;
    const int64_t ns = n >> p.sshift;
    if (n <= p.keep_all_n || ns <= p.rsel) {
        if (threadIdx.x == 0) p.tau_key[r] = 0u;
        return;
    }
    Group<4> G{(int)threadIdx.x, red};
    Selector<4, SEL_LOG2NB> sel{G, hist, vars};
    const int elim = (int)((ns + SEL_THREADS - 1) / SEL_THREADS);
    const uint32_t *src = p.dense + off * p.H + (int64_t)hl * n + ((int64_t)1 << p.sshift) - 1;
    uint32_t key[TAU_E];
#pragma unroll
    for (int e = 0; e < TAU_E; ++e) {
        const int64_t gi = e * SEL_THREADS + threadIdx.x;
        key[e] = e < elim && gi < ns ? src[gi << p.sshift] : 0u;
    }
    auto fe = [&](auto f) {
#pragma unroll
        for (int e = 0; e < TAU_E; ++e)
            if (e < elim) f(key[e], e * SEL_THREADS + threadIdx.x);
    };
    const Rule rule = sel.select(fe, [](uint32_t x) { return x; }, (uint32_t)elim * SEL_THREADS,
                                 (uint32_t)p.rsel);
    if (threadIdx.x == 0) p.tau_key[r] = rule.T;
}

constexpr int DF_E = 16;                    // keys per thread of the decode filter
constexpr int DF_KEYS = DF_E * 256;         // keys per decode-filter block

struct DecFilterParams {
    const uint32_t *dense;
    const int64_t *offs;
    int B, H;
    int64_t chunks;  // DF_KEYS-key chunks per row (longest sequence)
    const uint32_t *tau_key;
    uint2 *surv;  // (row, half) streams of (float bits, key index), stride apart
    int *cnt;     // per (row, half): survivors found (may exceed cap_half)
    int cap_half, stride;
};

// Block = (row, chunk of DF_KEYS keys), coalesced reads of the row's score
// keys. Keys >= the row's threshold leave as survivors: even key indices to
// the row's first half stream, odd ones to the second (so a row that keeps
// every key splits evenly). One atomic per half and block claims the slots;
// slots past cap_half are not written (the count tells the selection).
__global__ void __launch_bounds__(256) k_dec_filter(DecFilterParams p) {
    __shared__ uint32_t wtot[2][4];
    __shared__ uint32_t base[2];
    const int64_t r = blockIdx.x / p.chunks;
    const int64_t c0 = (blockIdx.x % p.chunks) * (int64_t)DF_KEYS;
    const int b = (int)(r % p.B);
    const int hl = (int)(r / p.B);
    const int64_t off = p.offs[b];
    const int64_t n = p.offs[b + 1] - off;
    if (c0 >= n) return;
    const uint32_t *keys = p.dense + off * p.H + (int64_t)hl * n;
    const uint32_t T = p.tau_key[r];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, half = tid & 1;
    uint32_t key[DF_E];
#pragma unroll
    for (int e = 0; e < DF_E; ++e) {
        const int64_t c = c0 + e * 256 + tid;
        key[e] = c < n ? keys[c] : 0u;
    }
    auto keep = [&](int e) { return c0 + e * 256 + tid < n && key[e] >= T; };
    const uint64_t hmask = half ? 0xAAAAAAAAAAAAAAAAull : 0x5555555555555555ull;
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < DF_E; ++e) tot += __popcll(__ballot(keep(e)) & hmask);
    if (l < 2) wtot[l][w] = tot;
    __syncthreads();
    if (tid < 2) {
        const uint32_t t = wtot[tid][0] + wtot[tid][1] + wtot[tid][2] + wtot[tid][3];
        base[tid] = t ? (uint32_t)atomicAdd(&p.cnt[2 * r + tid], (int)t) : 0u;
    }
    __syncthreads();
    uint32_t pos = base[half];
    for (int v = 0; v < w; ++v) pos += wtot[half][v];
    uint2 *dst = p.surv + (2 * r + half) * (int64_t)p.stride;
    const uint64_t below = (1ull << l) - 1ull;
#pragma unroll
    for (int e = 0; e < DF_E; ++e) {
        const bool k = keep(e);
        const uint64_t m = __ballot(k) & hmask;
        if (k) {
            const uint32_t slot = pos + (uint32_t)__popcll(m & below);
            if (slot < (uint32_t)p.cap_half)
                dst[slot] = make_uint2(__float_as_uint(key_score(key[e])), (uint32_t)(c0 + e * 256 + tid));
        }
        pos += (uint32_t)__popcll(m);
    }
}

// ----------------------------------------------------------------- refine

struct RefParams {
    const void *q;
    const void *K;
    const uint32_t *cand;  // (groups, Kc) candidate lists
    int64_t Kc;            // list stride (K)
    int H, h0;             // heads of the tensors, first head of this pass
    int Hc;                // heads in this pass
    int64_t NG;            // groups per head (prefill: G; decode: B)
    int g;
    int64_t S;             // prefill sequence length
    int decode;
    const int64_t *offs;   // decode sequence offsets
    int nqw;               // queries (wavefronts) per block
    int nqb;               // blocks per group
    int top_k;
    int reg_bytes;         // per-wave LDS region
    int ref_cap;           // staged entries of the fused select (top_k + slack)
    int pad_first;         // literal per-position Refine: position 0 is padding
    int32_t *out_idx;
    float *out_score;
    // candidate sets larger than REF_MAXK: the gather writes every member's
    // candidate scores (orderable keys) to row (group * g + member) of gsc,
    // gstride words apart, and k_rowsel selects from there
    uint32_t *gsc;
    int64_t gstride;
};

// One block per (group, block of <= 8 member queries): gathers the keys of
// the group's candidate list, scores them against the member queries on MFMA
// (16x16: 16 candidates x 16 query columns, members in the first columns)
// into LDS, then every wavefront selects and orders its own query's top_k.
// ---- fused bucket select + sort of one wavefront's keys ----------------
// Exact selection and ordering (score desc, key index asc) of the msel best
// of nc keys held by a wavefront, position 256 e + 4 l + v in key[4 e + v]
// of lane l (key 0 = empty slot, below every score). idx_of(pos) gives the
// key index of a position (any pos < 2^POSB must be safe to pass); smp is
// one key of the list per lane, taken evenly over it.
// 1. The lower end of the coarse range is a sampled key that lies below
//    the msel-th best with high probability (the r-th largest of 64 keys
//    taken evenly from the list, r four standard deviations past the
//    rank the msel-th key is expected to have among them); when fewer
//    than msel keys reach it, the list minimum. Bins over [lower end,
//    max] then spread the keys that matter (score tails and keys below
//    zero would otherwise crowd them into a few bins, and the atomics of
//    a histogram pass would serialise on those addresses). A coarse
//    histogram (1024 bins) finds the bin holding the msel-th best key.
// 2. Equi-depth refinement: every coarse bin at or above it gets a
//    power-of-two number of fine buckets roughly proportional to its
//    count (2048 fine buckets in all, numbered from the best down), so a
//    fine bucket holds one or two keys on average whatever the shape of
//    the score distribution.
// 3. A fine histogram (32-bit counters in the staging area, free until
//    the scatter); its scan finds the fine bucket holding the msel-th key
//    and gives every fine bucket its output offset (16-bit, two a word).
// 4. Fine buckets up to that one are scattered as packed words (key bits
//    inside the bucket, position), tagged with their bucket.
// 5. Each lane takes a run of consecutive staged slots and ranks every
//    entry against its bucket companions (score desc, index asc).
// Out-of-range keys go to per-lane trash bins / slots: no branches, no
// single hot address (masking them off the LDS atomics measured slower).
// `my` is the wavefront's LDS region (REF_HDR bytes of header, then cap + 64
// staged words); positions take POSB bits of a staged word, key bits inside
// a fine bucket the other LOWB.
// Returns true when the row is out: either emit(row) was called with the
// row (key indices in final order) in row[0, msel) of LDS, or every entry
// went through put(rank, index) (ranks >= msel are not passed) and then
// emit(nullptr). Returns false when the general path must run; key[] then
// hold the keys again.
template <int E, int POSB, bool SMALLW, class IDX, class PUT, class EMIT>
__device__ __forceinline__ bool fused_select(uint32_t (&key)[E], const int e4, const int nc, const uint32_t msel,
                                             const uint32_t smp, unsigned char *my, const uint32_t cap, IDX idx_of,
                                             PUT put, EMIT emit) {
    constexpr int LOWB = 32 - POSB;
    constexpr uint32_t LM = (1u << LOWB) - 1u;
    constexpr uint32_t PM = (1u << POSB) - 1u;
    static_assert(64 * E <= (1 << POSB), "positions fit their bits");
    const int l = lane_id();
    constexpr int NC = 1 << REF_LOG2C;            // coarse bins
    constexpr int CPL = NC / 64;                  // coarse bins per lane
    uint32_t *h1 = (uint32_t *)my;                // coarse counts, then the table
    uint32_t *h2 = h1 + NC + 64;                  // fine counters, two per word
    uint32_t *vars = h2 + REF_NB / 2 + 64;
    uint32_t *buf = (uint32_t *)(my + REF_HDR);   // ref_cap staged entries
    uint32_t mx = 0u;
#pragma unroll
    for (int e = 0; e < E / 4; ++e)
        if (e < e4) {
#pragma unroll
            for (int v = 0; v < 4; ++v) mx = max(mx, key[4 * e + v]);
        }
    mx = wave_max(mx);
    // the smallest key (empty slots, 0, wrap to the top): only when the
    // sampled lower end is not used or not below the msel-th key
    auto min_key = [&]() -> uint32_t {
        uint32_t mnm1 = 0xFFFFFFFFu;
#pragma unroll
        for (int e = 0; e < E / 4; ++e)
            if (e < e4) {
#pragma unroll
                for (int v = 0; v < 4; ++v) mnm1 = min(mnm1, key[4 * e + v] - 1u);
            }
        return wave_min(mnm1) + 1u;
    };
    uint32_t klo;
    {
        const float pf = (float)msel / (float)nc;
        const int rs = (int)ceilf(64.f * pf + 4.f * sqrtf(64.f * pf * (1.f - pf))) + 2;
        if (nc >= 64 && rs <= 64) {
            // the rs-th largest sample: a bitonic sort of the 64 samples,
            // largest in lane 0
            uint32_t v = smp;
#pragma unroll
            for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
                for (int jj = k >> 1; jj > 0; jj >>= 1) {
                    const uint32_t o = (uint32_t)__shfl_xor((int)v, jj);
                    const bool keep_max = ((l & k) == 0) == ((l & jj) == 0);
                    v = keep_max ? max(v, o) : min(v, o);
                }
            }
            klo = (uint32_t)__builtin_amdgcn_readlane((int)v, rs - 1);
        } else {
            klo = min_key();
        }
    }
    // lane l owns coarse bins [NC - CPL (l + 1), NC - CPL l), the top first
    uint32_t *mine = h1 + NC - CPL * (l + 1);
    uint32_t cc[CPL];
    int sh1 = 0;
    uint32_t b1 = 0, nt = 0;
    for (int att = 0; att < 2; ++att) {
        const int bw1 = bit_width(mx - klo);
        sh1 = bw1 > REF_LOG2C ? bw1 - REF_LOG2C : 0;
        // the coarse counts and trash bins (h2 is written before it is read)
        for (int i = l; i < (NC + 64) / 4; i += 64) ((uint4 *)h1)[i] = make_uint4(0u, 0u, 0u, 0u);
        if (l == 0) vars[0] = 0xFFFFFFFFu;
        wave_lds_sync();
#pragma unroll
        for (int e = 0; e < E / 4; ++e)
            if (e < e4) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t k = key[4 * e + v];
                    atomicAdd(&h1[k >= klo ? (k - klo) >> sh1 : (uint32_t)(NC + l)], 1u);
                }
            }
        wave_lds_sync();
        uint32_t loc = 0;
#pragma unroll
        for (int i = 0; i < CPL / 4; ++i) {
            const uint4 c4 = *(const uint4 *)(mine + 4 * i);
            cc[4 * i + 0] = c4.x;
            cc[4 * i + 1] = c4.y;
            cc[4 * i + 2] = c4.z;
            cc[4 * i + 3] = c4.w;
            loc += c4.x + c4.y + c4.z + c4.w;
        }
        uint32_t run = wave_incl_scan(loc) - loc;
#pragma unroll
        for (int i = CPL - 1; i >= 0; --i) {
            if (run < msel && msel <= run + cc[i]) {
                vars[0] = (uint32_t)(NC - CPL * (l + 1) + i);
                vars[1] = run + cc[i];
            }
            run += cc[i];
        }
        wave_lds_sync();
        b1 = vars[0];
        nt = vars[1];
        if (b1 != 0xFFFFFFFFu) break;
        klo = min_key();  // the sample was not below the msel-th key
    }
    // -- 2. fine buckets per coarse bin: n = the power of two nearest to
    //    0.9 * count * 2048 / nt (rounded down instead when that
    //    overshoots 2048 in all), at least 2^(sh1 - 20) so that a key's
    //    bits inside its fine bucket fit LOWB bits, at most 2^sh1. The
    //    table has one 8-byte entry per bin at or above b1, r = bin - b1,
    //    at index r + r / 16 (a lane writes 16 consecutive bins: the gap
    //    spreads the lanes' stores over the banks): x = last fine bucket of
    //    the bin + (r << log2(n)),
    //    y = sub | fine base << 5, sub = sh1 - log2(n). A key k with
    //    rel = k - kb (kb = the lower end of bin b1) then has its fine
    //    bucket at x - (rel >> sub) and its bits inside it in the low sub
    //    bits of rel (an empty bin: sub 0, the running base).
    const uint32_t lgmin = sh1 > LOWB ? (uint32_t)(sh1 - LOWB) : 0u;
    const float scl = (float)(REF_NB * 9 / 10) / (float)nt;
    for (int round_down = 0; round_down < 2; ++round_down) {
        uint32_t lgs[CPL], loc = 0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t bin = NC - CPL * (l + 1) + i;
            const uint32_t c = cc[i];
            uint32_t lg = 0xFFu;  // no fine buckets
            if (bin >= b1 && c != 0u) {
                const uint32_t want = max(1u, (uint32_t)((float)c * scl));
                lg = (uint32_t)(31 - __clz((int)want));
                // nearest: round up when want >= 1.5 * 2^lg
                if (!round_down && 2u * want >= 3u << lg) ++lg;
                lg = min(lg, (uint32_t)sh1);
                lg = max(lg, lgmin);
                loc += 1u << lg;
            }
            lgs[i] = lg;
        }
        const uint32_t total = wave_sum(loc);
        if (total > (uint32_t)REF_NB && !round_down) continue;
        uint32_t run = wave_incl_scan(loc) - loc;
        wave_lds_sync();
        uint2 *tab = (uint2 *)h1;
        static_assert(8 * (NC + NC / 16) <= 4 * (NC + 64 + REF_NB / 2 + 64), "the table ends before vars");
#pragma unroll
        for (int i = CPL - 1; i >= 0; --i) {
            const uint32_t lg = lgs[i];
            const uint32_t bin = NC - CPL * (l + 1) + i;
            // empty bins at or above b1 take no bucket but keep the base
            // running, so bases never increase with the bin
            if (bin >= b1) {
                const uint32_t r = bin - b1;
                tab[r + (r >> 4)] = lg != 0xFFu
                                        ? make_uint2(run + (1u << lg) - 1u + (r << lg), ((uint32_t)sh1 - lg) | (run << 5))
                                        : make_uint2(0u, run << 5);
            }
            if (lg != 0xFFu) run += 1u << lg;
        }
        if (l == 63) vars[2] = run;  // fine buckets in use
        break;
    }
    wave_lds_sync();
    const uint32_t kb = klo + (b1 << sh1);  // lower end of bin b1
    const uint2 *tab = (const uint2 *)h1;
    // a packed word's coarse bin is the lowest bin at or above b1 whose
    // table base is <= its fine bucket (bases fall as bins rise)
    auto unpack = [&](uint32_t w) -> uint32_t {
        if (w == 0xFFFFFFFFu) return 0u;
        const uint32_t fb = w >> 20;
        uint32_t lo = 0, hi = NC - 1 - b1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if ((tab[mid + (mid >> 4)].y >> 5) <= fb) hi = mid;
            else lo = mid + 1;
        }
        const uint32_t t = tab[lo + (lo >> 4)].y;
        const uint32_t sub = t & 31u;
        const uint32_t lg = (uint32_t)sh1 - sub;
        const uint32_t top = (1u << lg) - 1u - (fb - (t >> 5));
        const uint32_t low = (top << sub) | (w & ((1u << sub) - 1u));
        return kb + (lo << sh1) + low;
    };
    // the 32-bit fine counters (and 64 trash counters) take the staging
    // area, free until the scatter
    if (vars[2] <= (uint32_t)REF_NB && cap >= (uint32_t)REF_NB) {
        // packed word of a key: fine bucket << 20 | its bits inside the
        // fine bucket (0 = best bucket); 0xFFFFFFFF when not wanted
        // (below the range, below b1, or an empty slot). f = the counter
        // the key goes to: its fine bucket, or the lane's trash counter.
        const uint32_t trash_f = (uint32_t)(REF_NB + l);
        // every wanted key has kb <= k <= mx: one unsigned compare of
        // k - kb (keys below kb wrap past mx - kb)
        const uint32_t span = mx - kb;
        const uint32_t rmax = (uint32_t)(NC - 1) - b1;
        uint32_t *fc = buf;
        for (int i = l; i < (REF_NB + 64) / 4; i += 64) ((uint4 *)fc)[i] = make_uint4(0u, 0u, 0u, 0u);
        wave_lds_sync();
        // packed word of a key from rel = k - kb and its table entry t
        auto packed = [&](uint32_t rel, uint2 t, uint32_t &f) -> uint32_t {
            // sub = the low 5 bits of t.y, which is all the shift and the
            // bit-field extract read of it
            const uint32_t fb = t.x - (rel >> (t.y & 31u));
            const uint32_t w = (fb << 20) | __builtin_amdgcn_ubfe(rel, 0u, t.y);
            const bool ok = rel <= span;
            f = ok ? fb : trash_f;
            return ok ? w : 0xFFFFFFFFu;
        };
        uint32_t cmax;  // largest count of the buckets up to fstar this lane scans
        // -- 3. fine histogram, crossing, offsets. From here on each key
        //    register holds its packed word (every slot, so empty ones
        //    read as "not wanted" in all passes); unpack() gives the key
        //    back to the general path. With SLOTS, the counter's old value
        //    is the key's slot inside its fine bucket: sub[k / 4] keeps it,
        //    four 8-bit ones a word, for the scatter (rows whose staged
        //    buckets reach 256 keys take the general path); without, the
        //    scatter claims slots with atomics of its own (96 keys a lane
        //    leave no registers for the slots; lists of at most 1024 keys
        //    measured faster with the claims).
        //    Eight keys at a time: their eight table reads are issued
        //    before any of them is used, so that the batch waits for one
        //    LDS round trip, not eight; a batch's slots are taken into sub
        //    after the next batch's table reads have returned (LDS
        //    operations of a wavefront complete in order), so that they
        //    cost no wait of their own.
        static_assert(E % 8 == 0, "keys go in batches of eight");
        constexpr bool SLOTS = E <= 64 && !SMALLW;
        uint32_t sub[SLOTS ? E / 4 : 1];
        uint32_t got[8] = {};
        // the low bytes of four counts (a count of a bucket that is not
        // staged may pass 255: only its own byte may hold garbage)
        auto keep_slots = [&](int b) {
            if constexpr (SLOTS) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint32_t lo = __builtin_amdgcn_perm(got[4 * i + 1], got[4 * i], 0x0c0c0400u);
                    const uint32_t hi = __builtin_amdgcn_perm(got[4 * i + 3], got[4 * i + 2], 0x0c0c0400u);
                    sub[2 * b + i] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                }
            }
        };
#pragma unroll
        for (int e0 = 0; e0 < E / 4; e0 += 2) {
            if (e0 < e4) {
                uint32_t rel[8];
                uint2 t[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) rel[i] = key[4 * e0 + i] - kb;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t r = min(rel[i] >> sh1, rmax);
                    t[i] = tab[r + (r >> 4)];
                }
                __builtin_amdgcn_sched_barrier(0);
                if (e0 >= 2) keep_slots(e0 / 2 - 1);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (e0 + i / 4 < e4) {
                        uint32_t f;
                        key[4 * e0 + i] = packed(rel[i], t[i], f);
                        if constexpr (SLOTS) got[i] = atomicAdd(&fc[f], 1u);
                        else atomicAdd(&fc[f], 1u);
                    } else {
                        key[4 * e0 + i] = 0xFFFFFFFFu;
                    }
                }
            } else {
                if (e0 >= 2) keep_slots(e0 / 2 - 1);
#pragma unroll
                for (int i = 0; i < 8; ++i) key[4 * e0 + i] = 0xFFFFFFFFu;
            }
            __builtin_amdgcn_sched_barrier(0);  // bound the loads in flight
        }
        keep_slots(E / 8 - 1);
        wave_lds_sync();
        // lane l: fine buckets 32 l .. 32 l + 31; their output offsets,
        // two 16-bit ones a word, stay in registers until the scatter
        // path is taken (they go to h2, over the table)
        constexpr int OW = REF_NB / 128;
        uint32_t ow[OW];
        {
            const uint4 *fw = (const uint4 *)(fc + (REF_NB / 64) * l);
            uint32_t cnt[REF_NB / 64];
            uint32_t loc = 0;
            cmax = 0u;
#pragma unroll
            for (int i = 0; i < REF_NB / 256; ++i) {
                const uint4 c4 = fw[i];
                cnt[4 * i + 0] = c4.x;
                cnt[4 * i + 1] = c4.y;
                cnt[4 * i + 2] = c4.z;
                cnt[4 * i + 3] = c4.w;
                loc += c4.x + c4.y + c4.z + c4.w;
            }
            uint32_t run = wave_incl_scan(loc) - loc;
#pragma unroll
            for (int t = 0; t < REF_NB / 64; ++t) {
                const uint32_t c = cnt[t];
                if (run < msel) cmax = max(cmax, c);  // buckets 0 .. fstar only
                if (t & 1) ow[t >> 1] |= run << 16;
                else ow[t >> 1] = run;
                if (run < msel && msel <= run + c) {
                    vars[3] = (uint32_t)((REF_NB / 64) * l + t);
                    vars[4] = run + c;
                }
                run += c;
            }
        }
        wave_lds_sync();
        const uint32_t fstar = vars[3];
        const uint32_t nsc = vars[4];
        const uint32_t bmax = wave_max(cmax);  // the largest staged bucket
        // h1 (the table, dead once every key is packed) then holds a 16-bit
        // bucket tag per staged entry; h2 the buckets' 16-bit start
        // offsets.
        constexpr uint32_t STG = (uint32_t)(NC + 64 + REF_NB / 2 + 64);
        constexpr uint32_t TAGS = 2u * (uint32_t)(NC + 64) - 64u;  // + 64 trash tags
        constexpr int NSL = 36;                                     // staged slots per lane
        static_assert(NSL % 4 == 0 && 64 * NSL >= (int)TAGS, "every staged slot has a lane");
        if (nsc <= cap && nsc <= TAGS && msel <= STG && cap + 64u >= 64u * (uint32_t)NSL && (!SLOTS || bmax <= 255u)) {
#pragma unroll
            for (int i = 0; i < OW / 4; ++i)
                *(uint4 *)(h2 + OW * l + 4 * i) = make_uint4(ow[4 * i], ow[4 * i + 1], ow[4 * i + 2], ow[4 * i + 3]);
            wave_lds_sync();
            uint16_t *tag = (uint16_t *)h1;
            // bucket starts; without SLOTS the scatter's atomics advance
            // them to the bucket ends
            const uint16_t *start = (const uint16_t *)h2;
            // -- 4. scatter fine buckets 0 .. fstar as (key bits in the
            //    bucket << 12 | position) with the bucket as a tag, each
            //    to its bucket's start + its slot in the bucket (the eight
            //    start reads, or slot claims, of a batch are in flight
            //    together; keys not taken go to per-lane trash slots)
            if constexpr (!SLOTS) {
                const uint32_t trashf = (uint32_t)(REF_NB + 2 * l);
#pragma clang loop unroll(full)
                for (int e0 = 0; e0 < E / 4; e0 += 2)
                    if (e0 < e4) {
                        uint32_t cl8[8], fb[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const uint32_t w = key[4 * e0 + i];
                            fb[i] = (w >> 20) > fstar ? trashf : (w >> 20);
                            cl8[i] = atomicAdd(&h2[fb[i] >> 1], 1u << ((fb[i] & 1u) << 4));
                        }
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const int e = e0 + i / 4, v = i % 4;
                            const bool take = fb[i] < (uint32_t)REF_NB && e < e4;
                            const uint32_t slot = (cl8[i] >> ((fb[i] & 1u) << 4)) & 0xFFFFu;
                            buf[take ? slot : cap + l] =
                                ((key[4 * e0 + i] & LM) << POSB) | (256u * (uint32_t)e + (uint32_t)(4 * l + v));
                            tag[take ? slot : TAGS + l] = (uint16_t)fb[i];
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
            } else {
#pragma clang loop unroll(full)
                for (int e0 = 0; e0 < E / 4; e0 += 2)
                    if (e0 < e4) {
                        uint32_t fb[8], st[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            // a word of a key not wanted (all ones) has bucket
                            // 4095, past every fine bucket
                            fb[i] = key[4 * e0 + i] >> 20;
                            st[i] = start[min(fb[i], fstar)];
                        }
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const int k = 4 * e0 + i, e = e0 + i / 4, v = i % 4;
                            const bool take = fb[i] <= fstar && e < e4;
                            const uint32_t slot = st[i] + ((sub[k >> 2] >> (8 * (k & 3))) & 0xFFu);
                            buf[take ? slot : cap + l] =
                                ((key[k] & LM) << POSB) | (256u * (uint32_t)e + (uint32_t)(4 * l + v));
                            tag[take ? slot : TAGS + l] = (uint16_t)fb[i];
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
            }
            wave_lds_sync();
            // -- 5. rank inside the bucket. Slots run in bucket order, so
            //    ordering every bucket puts the row in place. Lane l
            //    holds the staged slots [W l, W (l + 1)) and X more on
            //    either side as 64-bit words (bucket + 1) << 52 |
            //    (inverted key bits in the bucket) << 32 | key index and
            //    runs odd-even transposition rounds until none swaps:
            //    the words of a bucket then stand in final order (score
            //    desc, index asc), and every bucket that touches the
            //    lane's own slots is whole in its window unless it
            //    reaches past an edge of the window. In that case every
            //    entry is ranked by a counted loop over its bucket
            //    instead and stored straight to the output row. Lists of
            //    at most 1024 keys (SMALLW) take W = 16, X = 16: their
            //    buckets of equal keys (integer-valued scores) run long,
            //    and the wider margins keep them inside the window; the
            //    others take W = NSL, X = 8.
            constexpr int W = SMALLW ? 16 : NSL;
            constexpr int X = SMALLW ? 16 : 8;
            // lane 1's left margin starts at slot 0 or later
            static_assert(W % 4 == 0 && X % 4 == 0 && X <= W, "margins in whole 16-byte pieces");
            constexpr int NW = W + 2 * X;
            const uint32_t s0 = (uint32_t)(W * l);
            const bool own = s0 < nsc;
            // window entries below lim hold slots before nsc
            const int lim = own ? (int)(nsc - s0) + X : 0;
            uint64_t A[NW];
            {
                const uint4 *bp = (const uint4 *)(buf + s0);
                const uint2 *tp = (const uint2 *)(tag + s0);
#pragma unroll
                for (int i = 0; i < W / 4; ++i) {
                    uint4 x = make_uint4(0u, 0u, 0u, 0u);
                    uint2 y = make_uint2(0u, 0u);
                    if (own) {
                        x = bp[i];
                        y = tp[i];
                    }
                    const int j = 4 * i + X;
                    const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
                    const uint32_t tg[4] = {y.x & 0xFFFFu, y.x >> 16, y.y & 0xFFFFu, y.y >> 16};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // window entry j + q is slot s0 - X + j + q; the list
                        // read stays inside LDS whatever the word holds
                        const uint32_t idx = idx_of(wd[q] & PM);
                        const uint32_t kv = ((tg[q] + 1u) << LOWB) | (LM - (wd[q] >> POSB));
                        A[j + q] = j + q < lim ? (((uint64_t)kv << 32) | idx) : ~0ull;
                    }
                }
                // the margins are the neighbours' own slots: the last X of
                // lane l - 1 (none left of lane 0: 0) and the first X of lane
                // l + 1 (none right of lane 63: all ones), across lanes by DPP
#pragma unroll
                for (int q = 0; q < X; ++q) {
                    const uint64_t a = A[W + q], b = A[X + q];
                    const uint32_t alo = dpp_zero<DPP_WAVE_SHR1>((uint32_t)a);
                    const uint32_t ahi = dpp_zero<DPP_WAVE_SHR1>((uint32_t)(a >> 32));
                    const uint32_t blo = dpp_u32<DPP_WAVE_SHL1>(~0u, (uint32_t)b);
                    const uint32_t bhi = dpp_u32<DPP_WAVE_SHL1>(~0u, (uint32_t)(b >> 32));
                    A[q] = ((uint64_t)ahi << 32) | alo;
                    A[X + W + q] = ((uint64_t)bhi << 32) | blo;
                }
            }
            // a bucket reaching from an own slot past the window
            const uint32_t tl = (uint32_t)(A[0] >> (32 + LOWB)), tf = (uint32_t)(A[X] >> (32 + LOWB));
            const uint32_t tb = (uint32_t)(A[X + W - 1] >> (32 + LOWB));
            const uint32_t tr = (uint32_t)(A[NW - 1] >> (32 + LOWB));
            const bool edge = own && ((tl != 0u && tl == tf) || (tb <= (uint32_t)REF_NB && tb == tr));
            // every staged slot has a lane (always so with SMALLW: nc <= 1024)
            const bool covered = !SMALLW || nsc <= 64u * (uint32_t)W;
            if (covered && __ballot(edge) == 0ull) {
                // entries only move inside their bucket, and odd-even
                // transposition orders m entries in m phases: ceil(bmax / 2)
                // rounds of both parities order every bucket (no test
                // round); more are never needed than the window holds
                const int rounds = (int)min((bmax + 1u) / 2u, (uint32_t)(NW / 2 + 1));
                for (int it = 0; it < rounds; ++it) {
#pragma unroll
                    for (int par = 0; par < 2; ++par) {
#pragma unroll
                        for (int i = par; i + 1 < NW; i += 2) {
                            const bool c = A[i] > A[i + 1];
                            const uint64_t a = A[i];
                            A[i] = c ? A[i + 1] : a;
                            A[i + 1] = c ? a : A[i + 1];
                        }
                    }
                }
                wave_lds_sync();
                // -- 6. finished row into LDS (every lane stores its whole
                //    run: slots past nsc are never read), then out with
                //    whole-line stores
#pragma unroll
                for (int t = 0; t < W; t += 4)
                    *(uint4 *)(buf + s0 + t) = make_uint4((uint32_t)A[X + t], (uint32_t)A[X + t + 1],
                                                          (uint32_t)A[X + t + 2], (uint32_t)A[X + t + 3]);
                wave_lds_sync();
                emit((const uint32_t *)buf);
                return true;
            }
            // staged entries u = l, l + 64, ...: every lane takes a share
            // whatever the staged count
            for (uint32_t u = (uint32_t)l; u < nsc; u += 64u) {
                {
                    const uint32_t w = buf[u];
                    const uint32_t f = tag[u];
                    uint32_t beg, end;
                    if constexpr (SLOTS) {
                        beg = start[f];
                        end = f < fstar ? (uint32_t)start[f + 1u] : nsc;
                    } else {
                        auto fend = [&](uint32_t b) { return (h2[b >> 1] >> ((b & 1u) << 4)) & 0xFFFFu; };
                        end = fend(f);
                        beg = f == 0u ? 0u : fend(f - 1u);
                    }
                    const uint32_t lw = w >> POSB;
                    const uint32_t myidx = idx_of(w & PM);
                    uint32_t rank = 0;
                    // four bucket companions per iteration: their LDS reads
                    // are in flight together (slots past the bucket are
                    // read inside the staging area and not counted)
                    for (uint32_t x = beg; x < end; x += 4u) {
                        uint32_t en[4], ix[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) en[i] = buf[min(x + (uint32_t)i, end - 1u)];
#pragma unroll
                        for (int i = 0; i < 4; ++i) ix[i] = idx_of(en[i] & PM);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t xi = x + (uint32_t)i;
                            const uint32_t le = en[i] >> POSB;
                            const bool in = xi < end && xi != u;
                            rank += (in && (le > lw || (le == lw && ix[i] < myidx))) ? 1u : 0u;
                        }
                    }
                    if (beg + rank < msel) put(beg + rank, myidx);
                }
            }
            emit((const uint32_t *)nullptr);
            return true;
        }
        // the boundary bucket does not fit: the general path needs the
        // keys back; keys below b1 rank under the msel-th and become 0.
#pragma unroll
        for (int i = 0; i < E; ++i) key[i] = unpack(key[i]);
    }
    wave_lds_sync();
    return false;
}

// ------------------------------------------------------- select (wave)

// One wavefront per row of sorted output (Reuse, dense): the row's survivors
// are loaded into registers as positions -- those of the first half, padded
// to a multiple of four, then those of the second -- and go through the
// fused bucket select; the best min(Ksel, n) in order go to every member row.
// Rows with more than 64 * SW_E positions, rows the fused path declines and
// calls that want scores are listed for k_select; overflowing rows are
// queued for k_fallback, as there.
__global__ void __launch_bounds__(64 * SW_WAVES) k_select_wave(SelParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int w = (int)(threadIdx.x >> 6), l = (int)(threadIdx.x & 63);
    const int64_t r = (int64_t)blockIdx.x * SW_WAVES + w;
    if (r >= p.rows) return;
    const int64_t j = r % p.G;
    const int hl = (int)(r / p.G);
    const int64_t n = sel_row_len(p, j);
    const int c0 = p.cnt[2 * r], c1 = p.cnt[2 * r + 1];
    const uint32_t msel = (uint32_t)min(p.Ksel, n);
    if (c0 > p.cap_half || c1 > p.cap_half || (uint32_t)(c0 + c1) < msel) {
        if (l == 0) {
            const uint32_t slot = atomicAdd(p.fb_count, 1u);
            p.fb_list[slot] = (uint32_t)r;
        }
        return;
    }
    auto to_list = [&]() {
        if (l == 0) {
            const uint32_t slot = atomicAdd(p.big_count, 1u);
            p.big_list[slot] = (uint32_t)r;
        }
    };
    const int ns = c0 + c1;
    const int c0p = (c0 + 3) & ~3;
    const int nv = c0p + c1;
    if (nv > 64 * SW_E || p.o.out_score) {
        to_list();
        return;
    }
    const uint2 *b0 = p.surv + (2 * r) * (int64_t)p.stride;
    const uint2 *b1 = b0 + p.stride;
    const int e4 = (nv + 255) / 256;
    uint32_t key[SW_E];
#pragma unroll
    for (int e = 0; e < SW_E / 4; ++e) {
        // positions pos .. pos + 3 lie in one half: lim of them are survivors
        const int pos = 256 * e + 4 * l;
        const int lim = pos < c0p ? c0 - pos : nv - pos;
        uint4 x0 = make_uint4(0u, 0u, 0u, 0u), x1 = x0;
        if (e < e4 && lim > 0) {
            const uint4 *src = (const uint4 *)(pos < c0p ? b0 + pos : b1 + (pos - c0p));
            x0 = src[0];
            x1 = src[1];
        }
        key[4 * e + 0] = 0 < lim ? score_key(__uint_as_float(x0.x)) : 0u;
        key[4 * e + 1] = 1 < lim ? score_key(__uint_as_float(x0.z)) : 0u;
        key[4 * e + 2] = 2 < lim ? score_key(__uint_as_float(x1.x)) : 0u;
        key[4 * e + 3] = 3 < lim ? score_key(__uint_as_float(x1.z)) : 0u;
    }
    uint32_t smp = 0u;
    if (ns >= 64) {
        const int s = (int)(((uint32_t)l * (uint32_t)ns) >> 6);
        smp = score_key(__uint_as_float(s < c0 ? b0[s].x : b1[s - c0].x));
    }
    // any position maps into this row's buffers (pads read stale words)
    auto idx_of = [&](uint32_t pos) -> uint32_t {
        const int q = min((int)pos, nv - 1);
        return q < c0p ? b0[q].y : b1[q - c0p].y;
    };
    const int64_t i0 = j * p.g;
    const int m = (int)min((int64_t)p.g, p.o.S - i0);
    const int64_t rstride = (int64_t)p.o.H * p.o.top_k;
    int32_t *dst0 = p.o.out_idx + (i0 * p.o.H + p.o.h0 + hl) * (int64_t)p.o.top_k;
    const bool done = fused_select<SW_E, 13, false>(
        key, e4, ns, msel, smp, smem + w * SW_REG, (uint32_t)SW_CAP, idx_of,
        [&](uint32_t fin, uint32_t idx) {
            for (int t = 0; t < m; ++t) dst0[t * rstride + fin] = (int32_t)idx;
        },
        [&](const uint32_t *row) {
            // the row's first msel & ~3 entries as 16-byte loads and stores
            // when the member rows are 16-byte aligned, the rest one by one
            int cs0 = row ? 0 : (int)msel;
            if (row && (p.o.top_k & 3) == 0 && ((uintptr_t)dst0 & 15u) == 0) {
                const int nv4 = (int)(msel & ~3u);
                for (int c = 4 * l; c < nv4; c += 256) {
                    const u32x4_t v = *(const u32x4_t *)(row + c);
                    // rows are not read again here: nontemporal stores
                    for (int t = 0; t < m; ++t) __builtin_nontemporal_store(v, (u32x4_t *)(dst0 + t * rstride + c));
                }
                cs0 = nv4;
            }
            for (int t = 0; t < m; ++t)
                for (int c = cs0 + l; c < p.o.top_k; c += 64)
                    dst0[t * rstride + c] = c < (int)msel ? (int32_t)row[c] : -1;
        });
    if (!done) to_list();
}

// LINES: key rows are gathered as whole 128-byte lines and rearranged into
// the MFMA layout in registers (bf16 blocks of several queries); otherwise
// the loads take the MFMA layout directly. GOUT: the scores go to global
// rows (p.gsc) and the kernel ends after the gather.
template <typename T, int D, bool LINES, bool GOUT, bool SMALLW>
__global__ void __launch_bounds__(512) k_refine(RefParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int nblk = (int)(p.NG * p.Hc) * p.nqb;
    const uint32_t L = xcd_remap(blockIdx.x, (uint32_t)nblk);
    const int64_t grp = L / p.nqb;
    const int qb = (int)(L % p.nqb);
    const int hl = (int)(grp / p.NG);
    const int64_t j = grp % p.NG;
    const int h = p.h0 + hl;
    int64_t qrow0, m, kbase, n;
    if (!p.decode) {
        qrow0 = j * p.g;
        m = min((int64_t)p.g, p.S - qrow0);
        kbase = 0;
        n = prefix_len(j, p.g);
    } else {
        qrow0 = j * p.g;
        m = p.g;
        kbase = p.offs[j];
        n = p.offs[j + 1] - kbase;
    }
    const int nc = (int)min(p.Kc, n);
    const int q0 = qb * p.nqw;
    const int nq = (int)min((int64_t)p.nqw, m - q0);
    // the wavefront index is uniform: held in scalar registers, so are the
    // addresses and counts derived from it
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int nthreads = p.nqw * 64;
    if (p.pad_first && qrow0 == 0) {
        // literal per-position Refine: no key precedes position 0
        const int64_t base = (int64_t)h * p.top_k;
        for (int c = tid; c < p.top_k; c += nthreads) {
            p.out_idx[base + c] = -1;
            if (p.out_score) p.out_score[base + c] = -INFINITY;
        }
        return;
    }

    uint32_t *cl = (uint32_t *)smem;                    // candidate list (Kc)
    unsigned char *regs = smem + ((p.Kc * 4 + 15) & ~15);
    const uint32_t *src = p.cand + grp * p.Kc;
    // eight loads a thread in flight before the first LDS store (a plain
    // copy loop waits for each load in turn)
    for (int i0 = tid; i0 < nc; i0 += 8 * nthreads) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[min(i0 + u * nthreads, nc - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * nthreads;
            if (i < nc) cl[i] = v[u];
        }
    }

    typedef typename std::conditional<std::is_same<T, float>::value, f32x4_t, bf16x8_t>::type frag_t;
    constexpr bool F32 = std::is_same<T, float>::value;
    constexpr int NKS = F32 ? D / 16 : D / 32;
    const T *Q = (const T *)p.q;
    const T *Kx = (const T *)p.K;
    const int qcol = l & 15, lq = l >> 4;
    frag_t bq[NKS];
    for (int ks = 0; ks < NKS; ++ks) {
        if (qcol < nq) {
            const int dofs = F32 ? 16 * ks + 4 * lq : 32 * ks + 8 * lq;
            bq[ks] = *(const frag_t *)(Q + ((qrow0 + q0 + qcol) * p.H + h) * (int64_t)D + dofs);
        } else {
            bq[ks] = frag_t{};
        }
    }
    __syncthreads();

    // gather + MFMA, four 16-candidate blocks per step so that 4*NKS row
    // loads per lane are in flight together
    const int nblocks = (nc + 15) / 16;
    // a list entry is always a key of the prefix; past the list the slot
    // holds stale LDS words: the clamp keeps every gather inside the tensor,
    // and scores past nc are never read
    auto mfma_store = [&](int b0, const frag_t (&a)[4][NKS]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            f32x4_t acc = f32x4_t{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                if constexpr (F32) {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][ks][v], bq[ks][v], acc, 0, 0, 0);
                } else {
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][ks], bq[ks], acc, 0, 0, 0);
                }
            }
            // lane holds query column qcol, candidates (b0+u)*16 + 4*lq + v
            // (a region has room for 64 scores past the last block)
            const int pp = (b0 + u) * 16 + 4 * lq;
            if (qcol < nq) {
                uint32_t *dst;
                if constexpr (GOUT) dst = p.gsc + (grp * p.g + q0 + qcol) * p.gstride + pp;
                else dst = (uint32_t *)(regs + qcol * p.reg_bytes) + pp;
                *(uint4 *)dst = make_uint4(score_key(acc[0]), score_key(acc[1]), score_key(acc[2]),
                                           score_key(acc[3]));
            }
        }
    };
    if constexpr (!LINES) {
        // MFMA-layout loads (16-byte pieces, lanes 16 apart): fp32, and
        // single-query blocks, whose many resident wavefronts hide the
        // latency better than the rearrangement below pays
        for (int b0 = 4 * w; b0 < nblocks; b0 += 4 * p.nqw) {
            frag_t a[4][NKS];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int pidx = (b0 + u) * 16 + qcol;
                const uint32_t c = min(cl[pidx], (uint32_t)(n - 1));
                const T *kr = Kx + ((kbase + c) * p.H + h) * (int64_t)D;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    a[u][ks] = *(const frag_t *)(kr + (F32 ? 16 * ks + 4 * lq : 32 * ks + 8 * lq));
            }
            mfma_store(b0, a);
        }
    } else {
        static_assert(!F32, "whole-line gathers are for bf16 keys");
        // Loads: 8 consecutive lanes read one whole 128-byte line of a key
        // row (the memory pipeline merges consecutive lanes only; the MFMA
        // layout would put 16 rows and 64 bytes of each in one load, as
        // 16-byte pieces of lanes 16 apart). Load (h, g), lane l: line h,
        // 16-byte chunk l & 7 of block row 2 (l >> 3) + g. The next step's
        // loads are issued before this step's rearrangement and MFMA.
        constexpr int NL = D / 64;  // 128-byte lines per key row
        typedef u32x4_t step_t[4][NL][2];
        auto load_step = [&](int b0, step_t &sv) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const int pidx = (b0 + u) * 16 + 2 * (l >> 3) + g;
                    const uint32_t c = min(cl[pidx], (uint32_t)(n - 1));
                    const T *kr = Kx + ((kbase + c) * p.H + h) * (int64_t)D + 8 * (l & 7);
#pragma unroll
                    for (int hh = 0; hh < NL; ++hh) sv[u][hh][g] = *(const u32x4_t *)(kr + 64 * hh);
                }
            }
        };
        // Into the MFMA layout (MFMA 2 h + q, lane 16 j + i: block row i,
        // chunk 4 q + j of line h): the two row halves trade across lane bit
        // 2 (DPP row shifts by 4), so that the register index becomes the
        // chunk's bit 2, then lane 16 j + i takes lane 4 i + j's word
        // (bpermute).
        const bool hi2 = (l & 4) != 0;
        const int from = (((l & 15) << 2) | (l >> 4)) << 2;
        auto compute_step = [&](int b0, const step_t &sv) {
            frag_t a[4][NKS];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int hh = 0; hh < NL; ++hh) {
                    u32x4_t t0, t1;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        // the shifts run on every lane (a DPP source lane
                        // must be active), then each lane picks
                        const uint32_t x0 = sv[u][hh][0][d], x1 = sv[u][hh][1][d];
                        const uint32_t up = dpp_zero<DPP_ROW_SHR4>(x1);
                        const uint32_t dn = dpp_zero<DPP_ROW_SHL4>(x0);
                        const uint32_t n0 = hi2 ? up : x0;
                        const uint32_t n1 = hi2 ? x1 : dn;
                        t0[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)n0);
                        t1[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)n1);
                    }
                    a[u][2 * hh] = __builtin_bit_cast(frag_t, t0);
                    a[u][2 * hh + 1] = __builtin_bit_cast(frag_t, t1);
                }
            }
            mfma_store(b0, a);
        };
        const int stride = 4 * p.nqw;
        step_t svA, svB;
        int b0 = 4 * w;
        if (b0 < nblocks) load_step(b0, svA);
        while (b0 < nblocks) {
            const int b1 = b0 + stride;
            if (b1 < nblocks) load_step(b1, svB);
            compute_step(b0, svA);
            if (b1 >= nblocks) break;
            const int b2 = b1 + stride;
            if (b2 < nblocks) load_step(b2, svA);
            compute_step(b1, svB);
            b0 = b2;
        }
    }
    if constexpr (GOUT) return;
    __syncthreads();
    if (w >= nq) return;

    // this wavefront's query: exact sorted top_k of its nc candidate scores.
    // Lane l holds positions 4*(e*64 + l) + v; slots past nc hold key 0,
    // below every score, so they never rank.
    unsigned char *my = regs + w * p.reg_bytes;
    const int e4 = (nc + 255) / 256;
    uint32_t key[REF_E];
#pragma unroll
    for (int e = 0; e < REF_E / 4; ++e) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (e < e4) v = *(const uint4 *)(my + (e * 64 + l) * 16);
        // position 256 e + 4 l + v; the bound is taken against a uniform
        // value so that no per-position register outlives the load (whole
        // chunks of 256 take no per-key test)
        const int rem = nc - 256 * e;
        if (rem >= 256) {
            key[4 * e + 0] = v.x;
            key[4 * e + 1] = v.y;
            key[4 * e + 2] = v.z;
            key[4 * e + 3] = v.w;
        } else {
            key[4 * e + 0] = 4 * l + 0 < rem ? v.x : 0u;
            key[4 * e + 1] = 4 * l + 1 < rem ? v.y : 0u;
            key[4 * e + 2] = 4 * l + 2 < rem ? v.z : 0u;
            key[4 * e + 3] = 4 * l + 3 < rem ? v.w : 0u;
        }
    }
    // one key of every 64th part of the list, for the coarse range below
    const uint32_t smp = nc >= 64 ? ((const uint32_t *)my)[((uint32_t)l * (uint32_t)nc) >> 6] : 0u;
    wave_lds_sync();
    const uint32_t msel = (uint32_t)min(p.top_k, nc);
    const int64_t obase = ((qrow0 + q0 + w) * p.H + h) * (int64_t)p.top_k;

    if (!p.out_score &&
        fused_select<REF_E, 12, SMALLW>(
            key, e4, nc, msel, smp, my, (uint32_t)p.ref_cap, [&](uint32_t pos) { return cl[pos]; },
            [&](uint32_t fin, uint32_t idx) { p.out_idx[obase + fin] = (int32_t)idx; },
            [&](const uint32_t *row) {
                // 16-byte loads and stores for the first msel & ~3 entries
                // when the output row is 16-byte aligned
                int32_t *dst = p.out_idx + obase;
                int cs0 = row ? 0 : (int)msel;
                if (row && ((uintptr_t)dst & 15u) == 0) {
                    const int nv4 = (int)(msel & ~3u);
                    // output rows are not read again here: nontemporal
                    // stores keep the cache for the candidate gathers
                    for (int c = 4 * l; c < nv4; c += 256)
                        __builtin_nontemporal_store(*(const u32x4_t *)(row + c), (u32x4_t *)(dst + c));
                    cs0 = nv4;
                }
                for (int c = cs0 + l; c < p.top_k; c += 64) dst[c] = c < (int)msel ? (int32_t)row[c] : -1;
            }))
        return;

    // ---- general path: the boundary bucket is too large to stage (heavy
    // ties); exact narrowing selection, then a bucket sort of the selection
    uint32_t *hist = (uint32_t *)my;                  // 1024 words
    uint32_t *vars = hist + (1 << REF_LOG2NB);
    uint32_t *red = vars + 8;
    uint32_t *bufk = red + 16;                        // top_k words
    uint16_t *bufp = (uint16_t *)(bufk + p.top_k);    // top_k positions
    Group<1> G{l, red};
    Selector<1, REF_LOG2NB> sel{G, hist, vars};
    auto fe = [&](auto f) {
#pragma unroll
        for (int e = 0; e < REF_E / 4; ++e)
            if (e < e4) {
#pragma unroll
                for (int v = 0; v < 4; ++v) f(key[4 * e + v], 256u * (uint32_t)e + (uint32_t)(4 * l + v));
            }
    };
    auto idx_of = [&](uint32_t pos) { return cl[pos]; };
    const Rule rule = msel >= (uint32_t)nc ? Rule{0u, 0u} : sel.select(fe, idx_of, (uint32_t)e4 * 256u, msel);
    auto fs = [&](auto f) {
#pragma unroll
        for (int e = 0; e < REF_E / 4; ++e)
            if (e < e4) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t k = key[4 * e + v];
                    const uint32_t pos = 256u * (uint32_t)e + (uint32_t)(4 * l + v);
                    bool take = k > rule.T;
                    if (k == rule.T) take = (~cl[pos]) >= rule.I;
                    if (k != 0u && take) f(k, pos);
                }
            }
    };
    sel.sort_selected(fs, idx_of, msel, bufk, bufp,
                      [&](uint32_t pos, uint32_t k, uint32_t pl) {
                          p.out_idx[obase + pos] = (int32_t)cl[pl];
                          if (p.out_score) p.out_score[obase + pos] = key_score(k);
                      });
    for (int pos = msel + l; pos < p.top_k; pos += 64) {
        p.out_idx[obase + pos] = -1;
        if (p.out_score) p.out_score[obase + pos] = -INFINITY;
    }
}

// Exact per-query top_k over candidate scores that a k_refine gather wrote
// to global rows (candidate sets larger than one wavefront's registers): one
// block per score row (group * g + member), RS_E scores per thread in
// registers, narrowing selection and bucket sort as in k_select. Slots past
// the list hold key 0, below every score.
__global__ void __launch_bounds__(SEL_THREADS) k_rowsel(RefParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *hist = (uint32_t *)smem;
    uint32_t *vars = hist + (1 << SEL_LOG2NB);
    uint32_t *red = vars + 8;
    uint32_t *bufk = red + 16;
    uint32_t *bufp = bufk + p.top_k;
    const int64_t r = blockIdx.x;
    const int u = (int)(r % p.g);
    const int64_t grp = r / p.g;
    const int hl = (int)(grp / p.NG);
    const int64_t j = grp % p.NG;
    const int h = p.h0 + hl;
    int64_t qrow0, m, n;
    if (!p.decode) {
        qrow0 = j * p.g;
        m = min((int64_t)p.g, p.S - qrow0);
        n = prefix_len(j, p.g);
    } else {
        qrow0 = j * p.g;
        m = p.g;
        n = p.offs[j + 1] - p.offs[j];
    }
    // members past a ragged group have no row; the literal mode's position
    // 0 was padded by k_refine
    if (u >= m || (p.pad_first && qrow0 == 0)) return;
    const int nc = (int)min(p.Kc, n);
    const uint32_t msel = (uint32_t)min((int64_t)p.top_k, (int64_t)nc);
    const uint32_t *keys = p.gsc + r * p.gstride;
    const uint32_t *cl = p.cand + grp * p.Kc;
    const int tid = threadIdx.x;
    uint32_t key[RS_E];
#pragma unroll
    for (int e = 0; e < RS_E; ++e) {
        const int pos = e * SEL_THREADS + tid;
        key[e] = pos < nc ? keys[pos] : 0u;
    }
    Group<4> G{tid, red};
    Selector<4, SEL_LOG2NB> sel{G, hist, vars};
    auto idx_of = [&](uint32_t pos) { return cl[pos]; };
    auto fe = [&](auto f) {
#pragma unroll
        for (int e = 0; e < RS_E; ++e) f(key[e], (uint32_t)(e * SEL_THREADS + tid));
    };
    const Rule rule = msel >= (uint32_t)nc ? Rule{0u, 0u}
                                           : sel.select(fe, idx_of, (uint32_t)(RS_E * SEL_THREADS), msel);
    auto fs = [&](auto f) {
#pragma unroll
        for (int e = 0; e < RS_E; ++e) {
            const uint32_t k = key[e];
            const uint32_t pos = (uint32_t)(e * SEL_THREADS + tid);
            // empty slots (key 0, past the list) never read the list
            if (k != 0u && (k > rule.T || (k == rule.T && (~cl[pos]) >= rule.I))) f(k, pos);
        }
    };
    const int64_t obase = ((qrow0 + u) * p.H + h) * (int64_t)p.top_k;
    sel.sort_selected(fs, idx_of, msel, bufk, bufp, [&](uint32_t pos, uint32_t k, uint32_t pl) {
        p.out_idx[obase + pos] = (int32_t)cl[pl];
        if (p.out_score) p.out_score[obase + pos] = key_score(k);
    });
    for (int pos = (int)msel + tid; pos < p.top_k; pos += SEL_THREADS) {
        p.out_idx[obase + pos] = -1;
        if (p.out_score) p.out_score[obase + pos] = -INFINITY;
    }
}

// ----------------------------------------------------- sparse attention

struct AttnParams {
    const void *q, *k, *v;   // (S, H, D)
    const int32_t *idx;      // (S, H, top_k); entries outside [0, S) are padding
    int64_t S;
    int H, top_k;
    float scale_log2;        // scale * log2(e)
    float *out;              // (S, H, D) float32
};

// Sum over the 16 lanes of a row, left in every lane of the row: DPP
// quad_perm [1,0,3,2] and [2,3,0,1], then row_half_mirror, then row_mirror.
__device__ __forceinline__ float row16_sum(float x) {
    auto step = [](float a, auto ctrl) {
        return a + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), decltype(ctrl)::value, 0xF, 0xF,
                                                              false));
    };
    x = step(x, std::integral_constant<int, 0xB1>{});
    x = step(x, std::integral_constant<int, 0x4E>{});
    x = step(x, std::integral_constant<int, 0x141>{});
    x = step(x, std::integral_constant<int, 0x140>{});
    return x;
}

// NE consecutive elements as float32 through 8- or 16-byte vector loads
template <typename T, int NE>
__device__ __forceinline__ void load_slice(const T *src, float (&x)[NE]) {
    if constexpr (std::is_same<T, float>::value) {
#pragma unroll
        for (int c = 0; c < NE / 4; ++c) {
            const float4 f = ((const float4 *)src)[c];
            x[4 * c] = f.x;
            x[4 * c + 1] = f.y;
            x[4 * c + 2] = f.z;
            x[4 * c + 3] = f.w;
        }
    } else {
        uint32_t wds[NE / 2];
        if constexpr (NE == 8) {
            const uint4 u = *(const uint4 *)src;
            wds[0] = u.x, wds[1] = u.y, wds[2] = u.z, wds[3] = u.w;
        } else {
            const uint2 u = *(const uint2 *)src;
            wds[0] = u.x, wds[1] = u.y;
        }
#pragma unroll
        for (int c = 0; c < NE / 2; ++c) {
            x[2 * c] = __uint_as_float(wds[c] << 16);
            x[2 * c + 1] = __uint_as_float(wds[c] & 0xFFFF0000u);
        }
    }
}

// Downstream sparse attention (the pages' quick-test attention, "Show Me
// The Code"): one wavefront per (head, position), consecutive positions of
// a head in consecutive wavefronts so that their shared index rows meet in
// L2. 16 lanes take one key/value row (D/16 elements each), 4 rows per
// instruction and 4 instructions in flight; the softmax runs online in base
// 2 (one rescale per 4 rows), the 4 row slots are merged at the end.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_sparse_attn(AttnParams p) {
    constexpr int NE = D / 16;             // elements per lane per row
    constexpr int U = 4;                   // rows per lane group in flight
    const int w = (int)(threadIdx.x >> 6), l = (int)(threadIdx.x & 63), j = l & 15, rr = l >> 4;
    const int64_t r = (int64_t)blockIdx.x * 4 + w;
    if (r >= p.S * p.H) return;
    const int h = (int)(r / p.S);
    const int64_t i = r % p.S;
    const int64_t rowq = (i * p.H + h) * (int64_t)D;
    float qv[NE];
    load_slice<T, NE>((const T *)p.q + rowq + NE * j, qv);
    const int32_t *ix = p.idx + (i * p.H + h) * (int64_t)p.top_k;
    const T *K = (const T *)p.k + (int64_t)h * D + NE * j;
    const T *V = (const T *)p.v + (int64_t)h * D + NE * j;
    const int64_t kstride = (int64_t)p.H * D;
    float m = -INFINITY, lsum = 0.f, acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.f;
    for (int t0 = 0; t0 < p.top_k; t0 += 4 * U) {
        int64_t c[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tt = t0 + 4 * u + rr;
            const int32_t cv = tt < p.top_k ? ix[tt] : -1;
            ok[u] = cv >= 0 && (int64_t)cv < p.S;
            c[u] = ok[u] ? cv : 0;
        }
        float kr[U][NE], vr[U][NE];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            load_slice<T, NE>(K + c[u] * kstride, kr[u]);
            load_slice<T, NE>(V + c[u] * kstride, vr[u]);
        }
        float sc[U], mn = m;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) d = fmaf(qv[e], kr[u][e], d);
            d = row16_sum(d) * p.scale_log2;
            sc[u] = ok[u] ? d : -INFINITY;
            mn = fmaxf(mn, sc[u]);
        }
        const float ref = mn == -INFINITY ? 0.f : mn;  // no valid entry yet: nothing to rescale
        const float a = exp2f(m - ref);
        lsum *= a;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] *= a;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float b = exp2f(sc[u] - ref);
            lsum += b;
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[e] = fmaf(b, vr[u][e], acc[e]);
        }
        m = mn;
    }
    // merge the 4 row slots: lanes j, j+16, j+32, j+48 hold the same dims
    float ma = fmaxf(m, __shfl_xor(m, 16));
    ma = fmaxf(ma, __shfl_xor(ma, 32));
    const float f = ma == -INFINITY ? 0.f : exp2f(m - ma);
    lsum *= f;
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        float x = acc[e] * f;
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        acc[e] = x;
    }
    if (rr == 0) {
        float *o = p.out + rowq + NE * j;
#pragma unroll
        for (int e = 0; e < NE; ++e) o[e] = lsum > 0.f ? acc[e] / lsum : 0.f;
    }
}

// ------------------------------------------- sparse attention, shared rows

constexpr int AG_NQ = 8;         // member queries per block
constexpr int AG_CH = 64;        // index-row entries per chunk
constexpr int AG_THREADS = 256;  // 4 wavefronts

struct AttnGroupParams {
    const void *q, *k, *v;   // (S, H, D)
    const int32_t *idx;      // (S, H, top_k); the row of position j*g serves group j
    int64_t S;
    int H, top_k, g;
    int64_t G;               // groups per head
    int nmb;                 // blocks per group (AG_NQ members each)
    float scale_log2;        // scale * log2(e)
    float *out;              // (S, H, D) float32
};

// Sparse attention for groups of g consecutive positions that share one
// index row (PIVOT-Reuse rows are the same for every member of a group):
// one block per (head, group, AG_NQ members) walks the row in chunks of
// AG_CH entries. The chunk's key and value rows are gathered once for all
// members into LDS (values as float32); scores come from MFMA 16x16 tiles
// (16 entries x 16 query columns, members in the first columns) and leave
// as base-2 logits; the softmax runs online per member (chunk maxima and
// sums through LDS); the weighted sum runs on the VALU, one thread per
// (member, D/32 dimensions). The next chunk's rows are loaded while the
// current one is reduced.
template <typename T, int D>
__global__ void __launch_bounds__(AG_THREADS) k_attn_group(AttnGroupParams p) {
    constexpr bool F32 = std::is_same<T, float>::value;
    constexpr int RB = D * (int)sizeof(T);       // bytes of a key row
    constexpr int RBP = RB + 16;                 // LDS stride of a key row (spreads the banks)
    constexpr int PER = RB / 4 / 16;             // 16-byte pieces per thread per row (4 threads a row)
    constexpr int DS = D / 32;                   // dimensions per thread in the weighted sum
    constexpr int VS = D + 4;                    // LDS stride (floats) of a value row (spreads the banks)
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *kt = smem;                                   // AG_CH key rows
    float *vt = (float *)(smem + AG_CH * RBP);                  // AG_CH value rows, float32
    float *ps = vt + AG_CH * VS;                                // [AG_NQ][AG_CH] probabilities
    float *wst = ps + AG_NQ * AG_CH;                            // [4][AG_NQ] wave maxima, [4][AG_NQ] sums

    const int nblk = (int)(p.G * p.H) * p.nmb;
    const uint32_t L = xcd_remap(blockIdx.x, (uint32_t)nblk);
    const int mb = (int)(L % p.nmb);
    const int64_t grp = L / p.nmb;
    const int h = (int)(grp / p.G);
    const int64_t j = grp % p.G;
    const int64_t i0 = j * p.g + (int64_t)mb * AG_NQ;           // first member of this block
    const int m = (int)min((int64_t)AG_NQ, min(j * p.g + p.g, p.S) - i0);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int qcol = l & 15, lq = l >> 4;
    const int pq = tid >> 5, sl = tid & 31;                     // weighted sum: member, dimension slice
    const T *Q = (const T *)p.q;
    const unsigned char *K = (const unsigned char *)p.k;
    const unsigned char *V = (const unsigned char *)p.v;
    const int64_t rstride = (int64_t)p.H * RB;                  // bytes between positions
    const int32_t *row = p.idx + ((j * p.g) * p.H + h) * (int64_t)p.top_k;

    // member queries as MFMA B fragments (column qcol), zero past m
    typedef typename std::conditional<F32, f32x4_t, bf16x8_t>::type frag_t;
    constexpr int NKS = F32 ? D / 16 : D / 32;
    frag_t bq[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (qcol < m) {
            const int dofs = F32 ? 16 * ks + 4 * lq : 32 * ks + 8 * lq;
            bq[ks] = *(const frag_t *)(Q + ((i0 + qcol) * p.H + h) * (int64_t)D + dofs);
        } else {
            bq[ks] = frag_t{};
        }
    }

    // chunk loads: thread t takes entry r = t / 4 of the chunk, quarter t % 4
    // of its key and value rows; two chunks are in flight (register sets A
    // and B, the chunk's parity)
    const int lr = tid >> 2, lp = tid & 3;
    struct ChunkRegs {
        u32x4_t k[PER], v[PER];
        bool valid;
    };
    auto load_chunk = [&](int c0, ChunkRegs &cr) {
        const int e = c0 + lr;
        const int32_t c = e < p.top_k ? row[e] : -1;
        cr.valid = c >= 0 && (int64_t)c < p.S;
        const int64_t off = (cr.valid ? (int64_t)c : 0) * rstride + (int64_t)h * RB + lp * (RB / 4);
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            cr.k[t] = *(const u32x4_t *)(K + off + 16 * t);
            cr.v[t] = *(const u32x4_t *)(V + off + 16 * t);
        }
    };
    // mrun / lrun / o: member pq's running maximum (base-2 logits), sum of
    // weights and weighted sum; mcol: member qcol's running maximum
    float mrun = -INFINITY, lrun = 0.f, mcol = -INFINITY, o[DS];
#pragma unroll
    for (int d = 0; d < DS; ++d) o[d] = 0.f;
    uint32_t *cvalid = (uint32_t *)(wst + 8 * AG_NQ);           // [AG_CH] entry valid flags
    ChunkRegs ra, rb;
    load_chunk(0, ra);
    if (AG_CH < p.top_k) load_chunk(AG_CH, rb);
    auto chunk = [&](int c0, ChunkRegs &cr) {
        // chunk into LDS
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            *(u32x4_t *)(kt + lr * RBP + lp * (RB / 4) + 16 * t) = cr.k[t];
            float *vd = vt + lr * VS + lp * (D / 4) + (16 / (int)sizeof(T)) * t;
            if constexpr (F32) {
                *(u32x4_t *)vd = cr.v[t];
            } else {
                const u32x4_t x = cr.v[t];
                *(float4 *)vd = make_float4(__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xFFFF0000u),
                                            __uint_as_float(x[1] << 16), __uint_as_float(x[1] & 0xFFFF0000u));
                *(float4 *)(vd + 4) = make_float4(__uint_as_float(x[2] << 16), __uint_as_float(x[2] & 0xFFFF0000u),
                                                  __uint_as_float(x[3] << 16), __uint_as_float(x[3] & 0xFFFF0000u));
            }
        }
        if (lp == 0) cvalid[lr] = cr.valid ? 1u : 0u;
        __syncthreads();
        // the chunk after next into the registers just emptied
        if (c0 + 2 * AG_CH < p.top_k) load_chunk(c0 + 2 * AG_CH, cr);
        // scores of entries 16 w .. 16 w + 15 for the member columns
        f32x4_t acc = f32x4_t{};
        {
            const unsigned char *kr = kt + (16 * w + qcol) * RBP;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                if constexpr (F32) {
                    const f32x4_t a = *(const f32x4_t *)(kr + (16 * ks + 4 * lq) * 4);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[v], bq[ks][v], acc, 0, 0, 0);
                } else {
                    const bf16x8_t a = *(const bf16x8_t *)(kr + (32 * ks + 8 * lq) * 2);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq[ks], acc, 0, 0, 0);
                }
            }
        }
        // lane (qcol, lq) holds entries 16 w + 4 lq + i of member qcol
        float sc[4], cm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 16 * w + 4 * lq + i;
            sc[i] = cvalid[e] ? acc[i] * p.scale_log2 : -INFINITY;
            cm = fmaxf(cm, sc[i]);
        }
        cm = fmaxf(cm, __shfl_xor(cm, 16));
        cm = fmaxf(cm, __shfl_xor(cm, 32));
        if (lq == 0 && qcol < AG_NQ) wst[w * AG_NQ + qcol] = cm;
        __syncthreads();
        // every thread keeps the running maximum of its own member (score
        // lanes: column qcol; weighted-sum threads: member pq) from the
        // chunk maxima of the four wavefronts
        auto chunk_max = [&](int q) {
            return fmaxf(fmaxf(wst[q], wst[AG_NQ + q]), fmaxf(wst[2 * AG_NQ + q], wst[3 * AG_NQ + q]));
        };
        const int qq = qcol < AG_NQ ? qcol : 0;
        mcol = fmaxf(mcol, chunk_max(qq));
        const float mnew = fmaxf(mrun, chunk_max(pq));
        {
            const float ref = mcol == -INFINITY ? 0.f : mcol;  // no valid entry yet: every p is 0
            float psum = 0.f, pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = exp2f(sc[i] - ref);
                psum += pv[i];
            }
            if (qcol < AG_NQ)
                *(float4 *)(ps + qcol * AG_CH + 16 * w + 4 * lq) = make_float4(pv[0], pv[1], pv[2], pv[3]);
            psum += __shfl_xor(psum, 16);
            psum += __shfl_xor(psum, 32);
            if (lq == 0 && qcol < AG_NQ) wst[4 * AG_NQ + w * AG_NQ + qcol] = psum;
        }
        __syncthreads();
        // weighted sum for member pq, dimensions DS * sl .. DS * sl + DS - 1
        {
            const float a = mrun == -INFINITY ? 0.f : exp2f(mrun - mnew);
            lrun = lrun * a + ((wst[4 * AG_NQ + pq] + wst[5 * AG_NQ + pq]) + (wst[6 * AG_NQ + pq] + wst[7 * AG_NQ + pq]));
            mrun = mnew;
#pragma unroll
            for (int d = 0; d < DS; ++d) o[d] *= a;
            const float *pr = ps + pq * AG_CH;
            const float *vr = vt + DS * sl;
#pragma unroll 4
            for (int e = 0; e < AG_CH; e += 4) {
                const float4 p4 = *(const float4 *)(pr + e);
                const float pe[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float *vv = vr + (e + u) * VS;
#pragma unroll
                    for (int d = 0; d < DS; ++d) o[d] = fmaf(pe[u], vv[d], o[d]);
                }
            }
        }
        __syncthreads();
    };
    for (int c0 = 0; c0 < p.top_k; c0 += 2 * AG_CH) {
        chunk(c0, ra);
        if (c0 + AG_CH < p.top_k) chunk(c0 + AG_CH, rb);
    }
    if (pq < m) {
        float *dst = p.out + ((i0 + pq) * p.H + h) * (int64_t)D + DS * sl;
        const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
#pragma unroll
        for (int d = 0; d < DS; ++d) dst[d] = lrun > 0.f ? o[d] * inv : 0.f;
    }
}

// ==================================================================== host

enum Stage { ST_PROXY = 0, ST_SAMPLE, ST_TAU, ST_SCAN, ST_SELECT, ST_FALLBACK, ST_REFINE,
             ST_DSCAN, ST_DSELECT, ST_COUNT };
static_assert(ST_COUNT == PIVOT_N_STAGES, "stage list matches the header");

constexpr int PROF_MAX = 8192;
struct ProfRec {
    int stage;
    hipEvent_t a, b;
};
bool g_prof_on = false;
thread_local bool t_prof_off = false;  // set while a call must record no events
int g_prof_used = 0;     // records filled since the last read
int g_prof_created = 0;  // records whose events exist
ProfRec g_prof[PROF_MAX];

// Records events around one kernel stage on `st` while profiling is on.
struct StageTimer {
    int slot = -1;
    hipStream_t st;
    StageTimer(int stage, hipStream_t s) : st(s) {
        if (!g_prof_on || t_prof_off || g_prof_used >= PROF_MAX) return;
        ProfRec &r = g_prof[g_prof_used];
        if (g_prof_used >= g_prof_created) {
            if (hipEventCreate(&r.a) != hipSuccess) return;
            if (hipEventCreate(&r.b) != hipSuccess) {
                (void)hipEventDestroy(r.a);
                return;
            }
            ++g_prof_created;
        }
        r.stage = stage;
        if (hipEventRecord(r.a, st) != hipSuccess) return;
        slot = g_prof_used++;
    }
    ~StageTimer() {
        if (slot >= 0) (void)hipEventRecord(g_prof[slot].b, st);
    }
};

struct Plan {
    int64_t S;
    int H, D, top_k, g, mode, dtype;
    bool dense;
    // literal per-position Refine: one scan row per position (g above is 1,
    // G is S), each row's proxy the mean of its group of gp positions
    bool literal;
    int gp;
    int64_t K, Ksel, G, n_max;
    int kstride;
    int64_t rsel;
    int cap_half, samp_half;
    int64_t keep_all_n;
    int n_tiles;
    size_t esz;
    int sel_e;       // survivors per thread of k_select (SEL_E or SEL_E_BIG)
    int buf_cap;     // entries of the selectors' LDS sort buffers
    int64_t gstride; // Refine with K > REF_MAXK: words per global score row (else 0)
    // per-head bytes of each workspace array
    size_t b_P, b_tau, b_cnt, b_scnt, b_surv, b_samp, b_cand, b_fbl, b_big, b_gsc;
    size_t fixed;  // fb_count + fallback scratch
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// the kernels move q, k and workspace data in 16-byte vectors
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int64_t pow2_floor(int64_t x) {
    int64_t p = 1;
    while (p * 2 <= x) p *= 2;
    return p;
}

int candidate_count(int32_t top_k, double ratio, int64_t *K) {
    if (top_k < 1 || !(ratio > 0.0) || !std::isfinite(ratio)) return PIVOT_EINVAL;
    const double prod = (double)top_k * ratio;
    if (!(prod < 9.0e18)) return PIVOT_EINVAL;
    const int64_t k = (int64_t)floor(prod);
    if (k < top_k) return PIVOT_EINVAL;
    *K = k;
    return PIVOT_OK;
}

// Threshold sampling of rows of up to n_max keys from which the best Ksel
// are wanted: every stride-th key is scored, tau is the rsel-th best sample.
// stride is a power of two giving about 64 expected samples above the
// Ksel-th best key (and at most 4080 samples per row, the registers of the
// threshold kernels); rsel puts tau four standard deviations (Poisson count
// of samples above the Ksel-th key) below it, so that at least Ksel keys
// score >= tau with overwhelming probability. A half stream of survivors
// holds cap_half: half the expected survivor count plus five standard
// deviations, plus four for the split between the halves. Rows of at most
// keep_all_n keys keep every key.
struct Sampling {
    int64_t stride, rsel, keep_all_n;
    int cap_half;
};

Sampling sampling(int64_t Ksel, int64_t n_max, int sel_e) {
    Sampling r;
    int64_t s = std::min<int64_t>(64, std::max<int64_t>(1, pow2_floor(std::max<int64_t>(1, Ksel / 64))));
    while ((n_max + s - 1) / s > 4096 - 16) s *= 2;
    r.stride = s;
    const double mu = (double)Ksel / (double)s;
    const double z = 4.0;
    const double root = (z + sqrt(z * z + 4.0 * mu)) / 2.0;
    r.rsel = (int64_t)ceil(root * root) + 1;
    const double X = (double)r.rsel * s, sig = sqrt((double)r.rsel) * s;
    int64_t ch = (int64_t)ceil((X + 5.0 * sig) / 2.0 + 4.0 * sqrt(X / 2.0)) + 16;
    ch = (ch + 63) / 64 * 64;
    ch = std::min<int64_t>(ch, (int64_t)sel_e * SEL_THREADS / 2);
    r.cap_half = (int)ch;
    r.keep_all_n = 2 * (int64_t)r.cap_half - 16;
    return r;
}

int make_plan(Plan &pl, int64_t S, int H, int D, int top_k, int g, double ratio, int mode,
              int dtype, bool dense) {
    if (S < 1 || S > (int64_t)INT32_MAX - 1 || H < 1 || g < 1) return PIVOT_EINVAL;
    if (dtype != PIVOT_F32 && dtype != PIVOT_BF16) return PIVOT_EINVAL;
    if (mode != PIVOT_REFINE && mode != PIVOT_REUSE && !(mode == PIVOT_REFINE_LITERAL && !dense))
        return PIVOT_EINVAL;
    if (top_k < 1) return PIVOT_EINVAL;
    int64_t K = top_k;
    if (!dense) {
        int rc = candidate_count(top_k, ratio, &K);
        if (rc) return rc;
    }
    if (D != 64 && D != 128) return PIVOT_EUNSUPPORTED;
    if (top_k > MAX_TOPK || K > MAX_K) return PIVOT_EUNSUPPORTED;
    pl.S = S;
    pl.H = H;
    pl.D = D;
    pl.top_k = top_k;
    pl.literal = mode == PIVOT_REFINE_LITERAL;
    pl.gp = g;
    pl.g = dense || pl.literal ? 1 : g;
    pl.mode = dense ? PIVOT_REUSE : (pl.literal ? PIVOT_REFINE : mode);
    pl.dtype = dtype;
    pl.dense = dense;
    pl.K = K;
    pl.Ksel = (pl.mode == PIVOT_REFINE) ? K : top_k;
    pl.G = (S + pl.g - 1) / pl.g;
    pl.n_max = std::max<int64_t>((pl.G - 1) * pl.g, 1);
    pl.esz = dtype == PIVOT_BF16 ? 2 : 4;
    pl.sel_e = pl.Ksel > SORT_MP * SEL_THREADS ? SEL_E_BIG : SEL_E;
    pl.buf_cap = (int)std::max<int64_t>(SORT_MP * SEL_THREADS, pl.Ksel);
    pl.gstride = pl.mode == PIVOT_REFINE && K > REF_MAXK ? ((K + 15) & ~(int64_t)15) + 64 : 0;
    const Sampling sm = sampling(pl.Ksel, pl.n_max, pl.sel_e);
    const int64_t s = sm.stride;
    pl.kstride = (int)s;
    pl.rsel = sm.rsel;
    pl.cap_half = sm.cap_half;
    pl.keep_all_n = sm.keep_all_n;
    // the scan addresses a key tile's rows by 32-bit offsets from the
    // tile's first key: SCAN_KEYS strided rows must span less than 4 GiB
    // (far beyond any input that fits one GPU's memory)
    if ((uint64_t)s * (uint64_t)H * (uint64_t)D * (uint64_t)pl.esz * SCAN_KEYS + (uint64_t)D * pl.esz >= (1ull << 32))
        return PIVOT_EUNSUPPORTED;
    const int64_t vmax = (pl.n_max + s - 1) / s;
    // a multiple of 8: every stream of the sample pass (4-byte scores)
    // starts on a 32-byte chunk, as the scan's flush addresses streams in
    // chunks of 8 entries
    pl.samp_half = (int)(((vmax + 1) / 2 + 8 + 7) & ~(int64_t)7);
    pl.n_tiles = (int)((pl.G + SCAN_ROWS - 1) / SCAN_ROWS);
    const size_t rows = (size_t)pl.G;
    pl.b_P = dense ? 0 : align256(rows * D * pl.esz);
    pl.b_tau = align256(rows * 4);
    pl.b_cnt = align256(rows * 8);
    pl.b_scnt = align256(rows * 8);
    pl.b_surv = align256(rows * 2 * (size_t)(pl.cap_half + 32) * 8);
    pl.b_samp = pl.n_max > pl.keep_all_n ? align256(rows * 2 * (size_t)(pl.samp_half + 32) * 4) : 0;
    pl.b_cand = pl.mode == PIVOT_REFINE ? align256(rows * (size_t)K * 4) : 0;
    pl.b_fbl = align256(rows * 4);
    pl.b_big = pl.mode == PIVOT_REUSE ? align256(rows * 4) : 0;
    pl.b_gsc = align256(rows * (size_t)pl.g * (size_t)pl.gstride * 4);
    pl.fixed = 256 + align256((size_t)FB_BLOCKS * (size_t)pl.n_max * 4);
    return PIVOT_OK;
}

size_t per_head_bytes(const Plan &pl) {
    return pl.b_P + pl.b_tau + pl.b_cnt + pl.b_scnt + pl.b_surv + pl.b_samp + pl.b_cand + pl.b_fbl + pl.b_big +
           pl.b_gsc;
}

hipError_t set_lds(const void *fn, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

#define HIP_TRY(x)                                    \
    do {                                              \
        if ((x) != hipSuccess) return PIVOT_EHIP;     \
    } while (0)

size_t sel_lds_bytes(int D, int buf_cap) {
    return ((size_t)(1 << SEL_LOG2NB) + 8 + 16 + 4 + 2 * (size_t)buf_cap) * 4 + (size_t)D * 4;
}

// k_select<false> (candidate lists) uses no staging buffers
size_t sel_cand_lds_bytes() { return ((size_t)(1 << SEL_LOG2NB) + 8 + 16 + 4) * 4; }

// LDS layout of k_refine: candidate list + one region per query wavefront.
// A region holds the query's scores first, then either the fused select
// (header + staged keys/positions) or the general selector's arrays; spare
// LDS becomes staging slack for the boundary bucket.
struct RefLayout {
    int nqw, reg_bytes, cap;
    size_t lds;
};
constexpr size_t LDS_MAX = 163840;

RefLayout refine_layout(int64_t K, int top_k, int g) {
    RefLayout L{};
    const size_t clb = ((size_t)K * 4 + 15) & ~(size_t)15;
    // scores of the whole list and 64 past its last 16-candidate block
    const size_t r_scores = (size_t)((K + 255) / 256) * 1024 + 256;
    const size_t r_general = ((size_t)(1 << REF_LOG2NB) + 8 + 16) * 4 + (size_t)top_k * 6;
    const size_t r_fused = (size_t)REF_HDR + 4 * ((size_t)top_k + 64 + 64);
    const size_t r_full = (size_t)REF_HDR + 4 * ((size_t)REF_FIX * 64 + 64);
    size_t need = std::max(r_scores, r_general);
    L.nqw = std::min(g, 8);
    // prefer room for the fused path; give up queries per block before it
    while (L.nqw > 1 && clb + (size_t)L.nqw * std::max(need, r_fused) > LDS_MAX) --L.nqw;
    size_t spare = ((LDS_MAX - clb) / (size_t)L.nqw) & ~(size_t)15;
    size_t r = std::min(spare, r_full);
    r = std::max(r, need);
    r = (r + 15) & ~(size_t)15;
    // regions 64 bytes past a multiple of 256 apart: the 16-byte score
    // stores of the query columns then fall in distinct LDS banks
    size_t r2 = (r & ~(size_t)255) + 64;
    if (r2 > r) r2 -= 256;
    if (r2 >= std::max(need, r_fused)) r = r2;
    L.reg_bytes = (int)r;
    // entries of the staging buffer, less the 64 trash slots at its end
    L.cap = r > (size_t)REF_HDR + 256 ? (int)std::min<size_t>((r - REF_HDR) / 4 - 64, (size_t)REF_FIX * 64) : 0;
    L.lds = clb + (size_t)L.nqw * r;
    return L;
}

template <typename T, int D, bool GOUT, bool SMALLW = false>
int launch_refine(const RefParams &rp, int nblocks, size_t lds, hipStream_t st) {
    if (sizeof(T) == 2 && rp.nqw > 1) {
        constexpr bool LINES = sizeof(T) == 2;
        HIP_TRY(set_lds((const void *)k_refine<T, D, LINES, GOUT, SMALLW>, lds));
        hipLaunchKernelGGL((k_refine<T, D, LINES, GOUT, SMALLW>), dim3(nblocks), dim3(64 * rp.nqw), lds, st, rp);
    } else {
        HIP_TRY(set_lds((const void *)k_refine<T, D, false, GOUT, SMALLW>, lds));
        hipLaunchKernelGGL((k_refine<T, D, false, GOUT, SMALLW>), dim3(nblocks), dim3(64 * rp.nqw), lds, st, rp);
    }
    HIP_TRY(hipGetLastError());
    return PIVOT_OK;
}

// Refine stage over rows groups (nqb blocks each). Candidate sets of up to
// REF_MAXK: k_refine gathers, scores and selects in one kernel (LDS layout
// from refine_layout). Larger sets: the gather writes the scores to rp.gsc
// and k_rowsel selects, one block per member row.
template <typename T>
int dispatch_refine(int D, RefParams rp, int64_t groups, int top_k, hipStream_t st) {
    if (rp.Kc <= REF_MAXK) {
        const RefLayout lay = refine_layout(rp.Kc, top_k, rp.g);
        rp.nqw = lay.nqw;
        rp.nqb = (rp.g + rp.nqw - 1) / rp.nqw;
        rp.reg_bytes = lay.reg_bytes;
        rp.ref_cap = lay.cap;
        const int nblocks = (int)(groups * rp.nqb);
        // lists of at most 1024 keys: the select's ranking window for
        // long runs of equal keys
        if (rp.Kc <= 1024)
            return D == 64 ? launch_refine<T, 64, false, true>(rp, nblocks, lay.lds, st)
                           : launch_refine<T, 128, false, true>(rp, nblocks, lay.lds, st);
        return D == 64 ? launch_refine<T, 64, false>(rp, nblocks, lay.lds, st)
                       : launch_refine<T, 128, false>(rp, nblocks, lay.lds, st);
    }
    rp.nqw = std::min(rp.g, 8);
    rp.nqb = (rp.g + rp.nqw - 1) / rp.nqw;
    rp.reg_bytes = 0;
    rp.ref_cap = 0;
    // the candidate list, and room for the reads of 64 slots past it
    const size_t lds = (((size_t)rp.Kc * 4 + 15) & ~(size_t)15) + 256;
    const int nblocks = (int)(groups * rp.nqb);
    int rc = D == 64 ? launch_refine<T, 64, true>(rp, nblocks, lds, st)
                     : launch_refine<T, 128, true>(rp, nblocks, lds, st);
    if (rc) return rc;
    const size_t rlds = ((size_t)(1 << SEL_LOG2NB) + 8 + 16 + 2 * (size_t)top_k) * 4;
    HIP_TRY(set_lds((const void *)k_rowsel, rlds));
    hipLaunchKernelGGL(k_rowsel, dim3((unsigned)(groups * rp.g)), dim3(SEL_THREADS), rlds, st, rp);
    HIP_TRY(hipGetLastError());
    return PIVOT_OK;
}

// Launches k_select (one block per row, or list mode when se.list) in the
// instance that holds Ksel's survivors.
int launch_select(const SelParams &se, bool sorted, int sel_e, unsigned blocks, hipStream_t st) {
    size_t lds = sorted ? sel_lds_bytes(0, se.buf_cap) : sel_cand_lds_bytes();
    const void *fn;
    if (sorted) fn = sel_e > SEL_E ? (const void *)k_select<true, SEL_E_BIG> : (const void *)k_select<true, SEL_E>;
    else fn = sel_e > SEL_E ? (const void *)k_select<false, SEL_E_BIG> : (const void *)k_select<false, SEL_E>;
    HIP_TRY(set_lds(fn, lds));
    if (sorted) {
        if (sel_e > SEL_E) hipLaunchKernelGGL((k_select<true, SEL_E_BIG>), dim3(blocks), dim3(SEL_THREADS), lds, st, se);
        else hipLaunchKernelGGL((k_select<true, SEL_E>), dim3(blocks), dim3(SEL_THREADS), lds, st, se);
    } else {
        if (sel_e > SEL_E) hipLaunchKernelGGL((k_select<false, SEL_E_BIG>), dim3(blocks), dim3(SEL_THREADS), lds, st, se);
        else hipLaunchKernelGGL((k_select<false, SEL_E>), dim3(blocks), dim3(SEL_THREADS), lds, st, se);
    }
    HIP_TRY(hipGetLastError());
    return PIVOT_OK;
}

template <typename T, int D, bool UNIT>
int launch_scan(const ScanParams &sp, hipStream_t st) {
    // dynamic LDS: the two key tiles (the survivor rings are static)
    const size_t lds = 2 * SCAN_KEYS * (size_t)D * sizeof(T);
    HIP_TRY(set_lds((const void *)k_scan<T, D, UNIT>, lds));
    hipLaunchKernelGGL((k_scan<T, D, UNIT>), dim3(sp.Hc * sp.n_tiles), dim3(SCAN_THREADS), lds, st, sp);
    HIP_TRY(hipGetLastError());
    return PIVOT_OK;
}

template <typename T>
int dispatch_scan(int D, const ScanParams &sp, hipStream_t st) {
    if (sp.kstride == 1) return D == 64 ? launch_scan<T, 64, true>(sp, st) : launch_scan<T, 128, true>(sp, st);
    return D == 64 ? launch_scan<T, 64, false>(sp, st) : launch_scan<T, 128, false>(sp, st);
}

template <typename T>
int run_prefill(const Plan &pl, const T *q, const T *k, int32_t *out_idx, float *out_score,
                unsigned char *ws, size_t ws_bytes, hipStream_t st) {
    const size_t phb = per_head_bytes(pl);
    if (ws_bytes < pl.fixed + phb) return PIVOT_EWORKSPACE;
    const int Hc_max = (int)std::min<size_t>((size_t)pl.H, (ws_bytes - pl.fixed) / phb);
    uint32_t *fb_count = (uint32_t *)ws;
    uint32_t *scratch = (uint32_t *)(ws + 256);
    unsigned char *base = ws + pl.fixed;
    const int64_t D = pl.D;

    for (int h0 = 0; h0 < pl.H; h0 += Hc_max) {
        const int Hc = std::min(Hc_max, pl.H - h0);
        const int64_t rows = (int64_t)Hc * pl.G;
        unsigned char *cur = base;
        auto take = [&](size_t per_head) {
            unsigned char *r = cur;
            cur += per_head * Hc;
            return r;
        };
        T *P = (T *)take(pl.b_P);
        float *tau = (float *)take(pl.b_tau);
        int *cnt = (int *)take(pl.b_cnt);
        int *scnt = (int *)take(pl.b_scnt);
        uint32_t *surv = (uint32_t *)take(pl.b_surv);
        uint32_t *samp = (uint32_t *)take(pl.b_samp);
        uint32_t *cand = (uint32_t *)take(pl.b_cand);
        uint32_t *fbl = (uint32_t *)take(pl.b_fbl);
        uint32_t *bigl = (uint32_t *)take(pl.b_big);
        uint32_t *gsc = (uint32_t *)take(pl.b_gsc);

        ScanParams sp{};
        if (pl.dense) {
            sp.P = q + (int64_t)h0 * D;
            sp.p_row = (int64_t)pl.H * D;
            sp.p_head = D;
        } else {
            const int64_t total = rows * D / (16 / (int64_t)sizeof(T));  // 16 bytes per thread
            const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
            StageTimer tm(ST_PROXY, st);
            hipLaunchKernelGGL((k_proxy<T>), dim3(blocks), dim3(256), 0, st, q, pl.S, pl.H, pl.D, pl.gp,
                               h0, Hc, pl.G, pl.literal ? pl.gp : 1, P);
            HIP_TRY(hipGetLastError());
            sp.P = P;
            sp.p_row = D;
            sp.p_head = pl.G * D;
        }
        sp.K = k;
        sp.k_row = (int64_t)pl.H * D;
        sp.k_head0 = (int64_t)h0 * D;
        sp.k_head = D;
        sp.G = pl.G;
        sp.g = pl.g;
        sp.n_tiles = pl.n_tiles;
        sp.Hc = Hc;
        hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, st, fb_count, (int64_t)2);
        HIP_TRY(hipGetLastError());

        // sample pass + thresholds
        if (pl.n_max > pl.keep_all_n) {
            ScanParams ss = sp;
            ss.kstride = pl.kstride;
            ss.koff = pl.kstride - 1;
            ss.tau = nullptr;
            ss.out = samp;
            ss.score_only = 1;
            ss.cap_half = pl.samp_half;
            ss.stride = pl.samp_half + 32;
            ss.cnt = scnt;
            ss.min_n = pl.keep_all_n;
            StageTimer tm(ST_SAMPLE, st);
            int rc = dispatch_scan<T>(pl.D, ss, st);
            if (rc) return rc;
        }
        {
            TauParams tp{samp, scnt, pl.samp_half, pl.samp_half + 32, tau, pl.G, pl.g, pl.keep_all_n, pl.rsel};
            const size_t lds = ((size_t)(1 << SEL_LOG2NB) + 8 + 16) * 4;
            StageTimer tm(ST_TAU, st);
            hipLaunchKernelGGL(k_tau, dim3((unsigned)rows), dim3(SEL_THREADS), lds, st, tp);
            HIP_TRY(hipGetLastError());
        }
        // main pass
        {
            ScanParams sm = sp;
            sm.kstride = 1;
            sm.koff = 0;
            sm.tau = tau;
            sm.out = surv;
            sm.cap_half = pl.cap_half;
            sm.stride = pl.cap_half + 32;
            sm.cnt = cnt;
            sm.min_n = 0;
            StageTimer tm(ST_SCAN, st);
            int rc = dispatch_scan<T>(pl.D, sm, st);
            if (rc) return rc;
        }
        RowOut ro{};
        ro.cand = cand;
        ro.K = pl.K;
        ro.out_idx = out_idx;
        ro.out_score = out_score;
        ro.top_k = pl.top_k;
        ro.H = pl.H;
        ro.h0 = h0;
        ro.S = pl.S;
        ro.g = pl.g;
        const int sorted_out = pl.mode == PIVOT_REUSE ? 1 : 0;
        {
            SelParams se{(const uint2 *)surv, cnt, pl.cap_half, pl.cap_half + 32, pl.G, pl.g, pl.Ksel, sorted_out, ro, fbl, fb_count};
            se.big_list = bigl;
            se.big_count = fb_count + 1;
            se.rows = rows;
            se.buf_cap = pl.buf_cap;
            StageTimer tm(ST_SELECT, st);
            // the wavefront sort stages at most 2112 entries: top_k up to
            // 2048 leaves the boundary bucket its slack
            if (sorted_out && pl.Ksel <= 2048) {
                const size_t wlds = (size_t)SW_WAVES * SW_REG;
                HIP_TRY(set_lds((const void *)k_select_wave, wlds));
                hipLaunchKernelGGL(k_select_wave, dim3((unsigned)((rows + SW_WAVES - 1) / SW_WAVES)),
                                   dim3(64 * SW_WAVES), wlds, st, se);
                HIP_TRY(hipGetLastError());
                se.list = 1;
                int rc = launch_select(se, true, pl.sel_e, (unsigned)std::min<int64_t>(rows, 2048), st);
                if (rc) return rc;
            } else {
                int rc = launch_select(se, sorted_out != 0, pl.sel_e, (unsigned)rows, st);
                if (rc) return rc;
            }
        }
        {
            FbParams fp{};
            fp.fb_list = fbl;
            fp.fb_count = fb_count;
            fp.P = sp.P;
            fp.p_row = sp.p_row;
            fp.p_head = sp.p_head;
            fp.K = k;
            fp.k_row = sp.k_row;
            fp.k_head0 = sp.k_head0;
            fp.k_head = sp.k_head;
            fp.G = pl.G;
            fp.g = pl.g;
            fp.scratch = scratch;
            fp.n_max = pl.n_max;
            fp.decode = 0;
            fp.Ksel = pl.Ksel;
            fp.sorted_out = sorted_out;
            fp.o = ro;
            fp.D = pl.D;
            fp.buf_cap = pl.buf_cap;
            const size_t lds = sel_lds_bytes(pl.D, pl.buf_cap);
            StageTimer tm(ST_FALLBACK, st);
            HIP_TRY(set_lds((const void *)k_fallback<T>, lds));
            hipLaunchKernelGGL((k_fallback<T>), dim3(FB_BLOCKS), dim3(SEL_THREADS), lds, st, fp);
            HIP_TRY(hipGetLastError());
        }
        if (pl.mode == PIVOT_REFINE) {
            RefParams rp{};
            rp.q = q;
            rp.K = k;
            rp.cand = cand;
            rp.Kc = pl.K;
            rp.H = pl.H;
            rp.h0 = h0;
            rp.Hc = Hc;
            rp.NG = pl.G;
            rp.g = pl.g;
            rp.S = pl.S;
            rp.decode = 0;
            rp.offs = nullptr;
            rp.top_k = pl.top_k;
            rp.pad_first = pl.literal ? 1 : 0;
            rp.out_idx = out_idx;
            rp.out_score = out_score;
            rp.gsc = gsc;
            rp.gstride = pl.gstride;
            StageTimer tm(ST_REFINE, st);
            int rc = dispatch_refine<T>(pl.D, rp, rows, pl.top_k, st);
            if (rc) return rc;
        }
    }
    return PIVOT_OK;
}

struct DecPlan {
    int B, g, H, D, top_k, mode, dtype;
    int64_t K, Ksel, total, max_ctx;
    size_t esz;
    Sampling sm;
    int sshift;
    int64_t chunks;
    int sel_e, buf_cap;
    int64_t gstride;
    size_t o_offs, o_P, o_dense, o_tau, o_cnt, o_surv, o_fbl, o_big, o_cand, o_gsc, bytes;
};

int make_dec_plan(DecPlan &dp, int B, const int64_t *ctx, int g, int H, int D, int top_k,
                  double ratio, int mode, int dtype) {
    if (B < 1 || g < 1 || H < 1 || top_k < 1 || !ctx) return PIVOT_EINVAL;
    if (dtype != PIVOT_F32 && dtype != PIVOT_BF16) return PIVOT_EINVAL;
    if (mode != PIVOT_REFINE && mode != PIVOT_REUSE) return PIVOT_EINVAL;
    int64_t K;
    int rc = candidate_count(top_k, ratio, &K);
    if (rc) return rc;
    int64_t total = 0, mx = 0;
    for (int b = 0; b < B; ++b) {
        if (ctx[b] < 1 || ctx[b] > (int64_t)INT32_MAX) return PIVOT_EINVAL;
        total += ctx[b];
        mx = std::max(mx, ctx[b]);
    }
    if ((int64_t)B * g > (int64_t)INT32_MAX) return PIVOT_EINVAL;
    if (D != 64 && D != 128) return PIVOT_EUNSUPPORTED;
    if (top_k > MAX_TOPK || K > MAX_K) return PIVOT_EUNSUPPORTED;
    dp.B = B;
    dp.g = g;
    dp.H = H;
    dp.D = D;
    dp.top_k = top_k;
    dp.mode = mode;
    dp.dtype = dtype;
    dp.K = K;
    dp.Ksel = mode == PIVOT_REFINE ? K : top_k;
    dp.total = total;
    dp.max_ctx = mx;
    dp.esz = dtype == PIVOT_BF16 ? 2 : 4;
    dp.sel_e = dp.Ksel > SORT_MP * SEL_THREADS ? SEL_E_BIG : SEL_E;
    dp.buf_cap = (int)std::max<int64_t>(SORT_MP * SEL_THREADS, dp.Ksel);
    dp.gstride = mode == PIVOT_REFINE && K > REF_MAXK ? ((K + 15) & ~(int64_t)15) + 64 : 0;
    dp.sm = sampling(dp.Ksel, mx, dp.sel_e);
    dp.sshift = 0;
    while (((int64_t)1 << dp.sshift) < dp.sm.stride) ++dp.sshift;
    dp.chunks = (mx + DF_KEYS - 1) / DF_KEYS;
    const size_t rows = (size_t)H * B;
    if ((int64_t)rows * dp.chunks > (int64_t)INT32_MAX) return PIVOT_EUNSUPPORTED;
    size_t off = 0;
    dp.o_offs = off;
    off += align256((size_t)(B + 1) * 8);
    dp.o_P = off;
    off += align256((size_t)H * B * D * dp.esz);
    dp.o_dense = off;
    off += align256((size_t)total * H * 4);
    dp.o_tau = off;
    off += align256(rows * 4);
    dp.o_cnt = off;  // 2 counts per row, then the fallback and list counters
    off += align256((rows * 2 + 2) * 4);
    dp.o_surv = off;
    off += align256(rows * 2 * (size_t)(dp.sm.cap_half + 32) * 8);
    dp.o_fbl = off;
    off += align256(rows * 4);
    dp.o_big = off;
    off += align256(rows * 4);
    dp.o_cand = off;
    off += mode == PIVOT_REFINE ? align256((size_t)H * B * K * 4) : 0;
    dp.o_gsc = off;
    off += align256((size_t)H * B * (size_t)g * (size_t)dp.gstride * 4);
    dp.bytes = off;
    return PIVOT_OK;
}

template <typename T, int D>
int launch_dec_scan(const DecScanParams &ds, int nblocks, int H, hipStream_t st) {
    (void)H;
    hipLaunchKernelGGL((k_decode_scan<T, D>), dim3(nblocks), dim3(DEC_THREADS), 0, st, ds);
    HIP_TRY(hipGetLastError());
    return PIVOT_OK;
}

template <typename T>
int run_decode(const DecPlan &dp, const int64_t *ctx, const T *q, const T *kc, int32_t *out_idx,
               float *out_score, unsigned char *ws, hipStream_t st) {
    int64_t *offs = (int64_t *)(ws + dp.o_offs);
    T *P = (T *)(ws + dp.o_P);
    uint32_t *dense = (uint32_t *)(ws + dp.o_dense);
    uint32_t *cand = (uint32_t *)(ws + dp.o_cand);
    uint32_t *tau_key = (uint32_t *)(ws + dp.o_tau);
    int *cnt = (int *)(ws + dp.o_cnt);
    uint2 *surv = (uint2 *)(ws + dp.o_surv);
    uint32_t *fbl = (uint32_t *)(ws + dp.o_fbl);
    uint32_t *bigl = (uint32_t *)(ws + dp.o_big);
    const int64_t rows = (int64_t)dp.H * dp.B;
    uint32_t *ctr = (uint32_t *)(cnt + 2 * rows);  // fallback count, list count
    // prefix offsets travel as kernel arguments, 64 per launch
    {
        int64_t run = 0;
        for (int s0 = 0; s0 <= dp.B; s0 += 64) {
            Offsets64 a{};
            a.start = s0;
            a.count = std::min(64, dp.B + 1 - s0);
            for (int t = 0; t < a.count; ++t) {
                const int b = s0 + t;
                if (b == 0) run = 0;
                a.v[t] = run;
                if (b < dp.B) run += ctx[b];
            }
            hipLaunchKernelGGL(k_put_offsets, dim3(1), dim3(64), 0, st, offs, a);
            HIP_TRY(hipGetLastError());
        }
    }
    {
        const int64_t total = (int64_t)dp.H * dp.B * dp.D / (16 / (int64_t)sizeof(T));  // 16 bytes per thread
        const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
        StageTimer tm(ST_PROXY, st);
        hipLaunchKernelGGL((k_proxy<T>), dim3(blocks), dim3(256), 0, st, q, (int64_t)dp.B * dp.g, dp.H,
                           dp.D, dp.g, 0, dp.H, (int64_t)dp.B, 1, P);
        HIP_TRY(hipGetLastError());
    }
    {
        DecScanParams ds{P, kc, offs, dp.B, dp.H, (dp.max_ctx + DEC_TOKENS - 1) / DEC_TOKENS, dense};
        const int nblocks = (int)((int64_t)dp.B * ((dp.H + 3) / 4) * ds.max_chunks);
        StageTimer tm(ST_DSCAN, st);
        int rc = dp.D == 64 ? launch_dec_scan<T, 64>(ds, nblocks, dp.H, st)
                            : launch_dec_scan<T, 128>(ds, nblocks, dp.H, st);
        if (rc) return rc;
    }
    RowOut ro{};
    ro.cand = cand;
    ro.K = dp.K;
    ro.out_idx = out_idx;
    ro.out_score = out_score;
    ro.top_k = dp.top_k;
    ro.H = dp.H;
    ro.h0 = 0;
    ro.S = (int64_t)dp.B * dp.g;
    ro.g = dp.g;
    const int sorted_out = dp.mode == PIVOT_REUSE ? 1 : 0;
    {
        const int64_t nz = 2 * rows + 2;
        hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)std::min<int64_t>((nz + 255) / 256, 1024)), dim3(256), 0,
                           st, (uint32_t *)cnt, nz);
        HIP_TRY(hipGetLastError());
        DecTauParams tp{dense, dp.sshift, offs, dp.B, dp.H, dp.sm.keep_all_n, dp.sm.rsel, tau_key};
        const size_t lds = ((size_t)(1 << SEL_LOG2NB) + 8 + 16) * 4;
        StageTimer tm(ST_TAU, st);
        hipLaunchKernelGGL(k_dec_tau, dim3((unsigned)rows), dim3(SEL_THREADS), lds, st, tp);
        HIP_TRY(hipGetLastError());
    }
    {
        StageTimer tm(ST_DSELECT, st);
        DecFilterParams fp{dense, offs, dp.B, dp.H, dp.chunks, tau_key, surv, cnt, dp.sm.cap_half,
                           dp.sm.cap_half + 32};
        hipLaunchKernelGGL(k_dec_filter, dim3((unsigned)(rows * dp.chunks)), dim3(256), 0, st, fp);
        HIP_TRY(hipGetLastError());
        SelParams se{surv, cnt, dp.sm.cap_half, dp.sm.cap_half + 32, (int64_t)dp.B, dp.g, dp.Ksel, sorted_out,
                     ro, fbl, ctr};
        se.big_list = bigl;
        se.big_count = ctr + 1;
        se.rows = rows;
        se.offs = offs;
        se.buf_cap = dp.buf_cap;
        if (sorted_out && dp.Ksel <= 2048) {
            const size_t wlds = (size_t)SW_WAVES * SW_REG;
            HIP_TRY(set_lds((const void *)k_select_wave, wlds));
            hipLaunchKernelGGL(k_select_wave, dim3((unsigned)((rows + SW_WAVES - 1) / SW_WAVES)),
                               dim3(64 * SW_WAVES), wlds, st, se);
            HIP_TRY(hipGetLastError());
            se.list = 1;
            int rc = launch_select(se, true, dp.sel_e, (unsigned)std::min<int64_t>(rows, 2048), st);
            if (rc) return rc;
        } else {
            int rc = launch_select(se, sorted_out != 0, dp.sel_e, (unsigned)rows, st);
            if (rc) return rc;
        }
    }
    {
        FbParams fp{};
        fp.fb_list = fbl;
        fp.fb_count = ctr;
        fp.decode = 1;
        fp.dense = dense;
        fp.offs = offs;
        fp.B = dp.B;
        fp.H = dp.H;
        fp.Ksel = dp.Ksel;
        fp.sorted_out = sorted_out;
        fp.o = ro;
        fp.D = dp.D;
        fp.buf_cap = dp.buf_cap;
        const size_t lds = sel_lds_bytes(dp.D, dp.buf_cap);
        StageTimer tm(ST_FALLBACK, st);
        HIP_TRY(set_lds((const void *)k_fallback<T>, lds));
        hipLaunchKernelGGL((k_fallback<T>), dim3((unsigned)std::min<int64_t>(rows, FB_BLOCKS)), dim3(SEL_THREADS),
                           lds, st, fp);
        HIP_TRY(hipGetLastError());
    }
    if (dp.mode == PIVOT_REFINE) {
        RefParams rp{};
        rp.q = q;
        rp.K = kc;
        rp.cand = cand;
        rp.Kc = dp.K;
        rp.H = dp.H;
        rp.h0 = 0;
        rp.Hc = dp.H;
        rp.NG = dp.B;
        rp.g = dp.g;
        rp.S = (int64_t)dp.B * dp.g;
        rp.decode = 1;
        rp.offs = offs;
        rp.top_k = dp.top_k;
        rp.out_idx = out_idx;
        rp.out_score = out_score;
        rp.gsc = (uint32_t *)(ws + dp.o_gsc);
        rp.gstride = dp.gstride;
        StageTimer tm(ST_REFINE, st);
        int rc = dispatch_refine<T>(dp.D, rp, (int64_t)dp.B * dp.H, dp.top_k, st);
        if (rc) return rc;
    }
    return PIVOT_OK;
}

// Device address of `scratch` on the current device, looked up on the
// first call on that device (with the device current) and kept.
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];

int static_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return PIVOT_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PIVOT_EHIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PIVOT_OK;
}

}  // namespace

// =================================================================== C ABI

extern "C" {

int pivot_sparse_attention(const void *q, const void *k, const void *v, int32_t dtype, int64_t S, int32_t H,
                           int32_t D, const int32_t *idx, int32_t top_k, float scale, float *out, void *stream) {
    if (!q || !k || !v || !idx || !out) return PIVOT_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(idx) || !aligned4(out)) return PIVOT_EINVAL;
    if (S < 1 || H < 1 || top_k < 1 || !std::isfinite(scale)) return PIVOT_EINVAL;
    if (dtype != PIVOT_F32 && dtype != PIVOT_BF16) return PIVOT_EINVAL;
    if (S > (int64_t)INT32_MAX) return PIVOT_EINVAL;
    if (D != 64 && D != 128) return PIVOT_EUNSUPPORTED;
    AttnParams ap{q, k, v, idx, S, H, top_k, scale * 1.4426950408889634f, out};
    const int64_t nblocks = (S * H + 3) / 4;
    if (nblocks > (int64_t)INT32_MAX) return PIVOT_EUNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == PIVOT_BF16) {
        if (D == 64) hipLaunchKernelGGL((k_sparse_attn<bf16_t, 64>), dim3((unsigned)nblocks), dim3(256), 0, st, ap);
        else hipLaunchKernelGGL((k_sparse_attn<bf16_t, 128>), dim3((unsigned)nblocks), dim3(256), 0, st, ap);
    } else {
        if (D == 64) hipLaunchKernelGGL((k_sparse_attn<float, 64>), dim3((unsigned)nblocks), dim3(256), 0, st, ap);
        else hipLaunchKernelGGL((k_sparse_attn<float, 128>), dim3((unsigned)nblocks), dim3(256), 0, st, ap);
    }
    return hipGetLastError() == hipSuccess ? PIVOT_OK : PIVOT_EHIP;
}

int pivot_sparse_attention_grouped(const void *q, const void *k, const void *v, int32_t dtype, int64_t S, int32_t H,
                                   int32_t D, const int32_t *idx, int32_t top_k, int32_t g, float scale, float *out,
                                   void *stream) {
    if (!q || !k || !v || !idx || !out) return PIVOT_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(idx) || !aligned4(out)) return PIVOT_EINVAL;
    if (S < 1 || H < 1 || top_k < 1 || g < 1 || !std::isfinite(scale)) return PIVOT_EINVAL;
    if (dtype != PIVOT_F32 && dtype != PIVOT_BF16) return PIVOT_EINVAL;
    if (S > (int64_t)INT32_MAX) return PIVOT_EINVAL;
    if (D != 64 && D != 128) return PIVOT_EUNSUPPORTED;
    AttnGroupParams ap{};
    ap.q = q;
    ap.k = k;
    ap.v = v;
    ap.idx = idx;
    ap.S = S;
    ap.H = H;
    ap.top_k = top_k;
    ap.g = g;
    ap.G = (S + g - 1) / g;
    ap.nmb = (g + AG_NQ - 1) / AG_NQ;
    ap.scale_log2 = scale * 1.4426950408889634f;
    ap.out = out;
    const int64_t nblocks = ap.G * H * ap.nmb;
    if (nblocks > (int64_t)INT32_MAX) return PIVOT_EUNSUPPORTED;
    const size_t esz = dtype == PIVOT_BF16 ? 2 : 4;
    const size_t lds = (size_t)AG_CH * (D * esz + 16) + (size_t)AG_CH * (D + 4) * 4 + (size_t)AG_NQ * AG_CH * 4 +
                       8 * AG_NQ * 4 + (size_t)AG_CH * 4;
    hipStream_t st = (hipStream_t)stream;
    auto go = [&](const void *fn, auto launch) -> int {
        HIP_TRY(set_lds(fn, lds));
        launch();
        return hipGetLastError() == hipSuccess ? PIVOT_OK : PIVOT_EHIP;
    };
    const dim3 grid((unsigned)nblocks), blk(AG_THREADS);
    if (dtype == PIVOT_BF16) {
        if (D == 64)
            return go((const void *)k_attn_group<bf16_t, 64>,
                      [&] { hipLaunchKernelGGL((k_attn_group<bf16_t, 64>), grid, blk, lds, st, ap); });
        return go((const void *)k_attn_group<bf16_t, 128>,
                  [&] { hipLaunchKernelGGL((k_attn_group<bf16_t, 128>), grid, blk, lds, st, ap); });
    }
    if (D == 64)
        return go((const void *)k_attn_group<float, 64>,
                  [&] { hipLaunchKernelGGL((k_attn_group<float, 64>), grid, blk, lds, st, ap); });
    return go((const void *)k_attn_group<float, 128>,
              [&] { hipLaunchKernelGGL((k_attn_group<float, 128>), grid, blk, lds, st, ap); });
}

const char *pivot_status_string(int status) {
    switch (status) {
    case PIVOT_OK: return "ok";
    case PIVOT_EINVAL: return "invalid argument";
    case PIVOT_EUNSUPPORTED: return "unsupported size or parameter";
    case PIVOT_EWORKSPACE: return "workspace too small";
    case PIVOT_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int pivot_candidate_count(int32_t top_k, double candidate_ratio, int64_t *K_out) {
    if (!K_out) return PIVOT_EINVAL;
    int64_t K;
    int rc = candidate_count(top_k, candidate_ratio, &K);
    if (rc) return rc;
    *K_out = K;
    return PIVOT_OK;
}

size_t pivot_prefill_workspace_bytes(int64_t S, int32_t H, int32_t D, int32_t top_k, int32_t g,
                                     double candidate_ratio, int32_t mode, int32_t dtype) {
    Plan pl;
    if (make_plan(pl, S, H, D, top_k, g, candidate_ratio, mode, dtype, false)) return 0;
    return pl.fixed + per_head_bytes(pl) * (size_t)H;
}

size_t dense_index_workspace_bytes(int64_t S, int32_t H, int32_t D, int32_t top_k, int32_t dtype) {
    Plan pl;
    if (make_plan(pl, S, H, D, top_k, 1, 1.0, PIVOT_REUSE, dtype, true)) return 0;
    return pl.fixed + per_head_bytes(pl) * (size_t)H;
}

static int prefill_common(const void *q, const void *k, int32_t dtype, int64_t S, int32_t H, int32_t D,
                          int32_t top_k, int32_t g, double ratio, int32_t mode, int32_t *out_idx,
                          float *out_score, void *workspace, size_t workspace_bytes, void *stream,
                          bool dense) {
    Plan pl;
    int rc = make_plan(pl, S, H, D, top_k, g, ratio, mode, dtype, dense);
    if (rc) return rc;
    if (!q || !k || !out_idx) return PIVOT_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned4(out_idx) || (out_score && !aligned4(out_score)))
        return PIVOT_EINVAL;
    if (!workspace || !aligned16(workspace)) return PIVOT_EWORKSPACE;
    if (workspace_bytes < pl.fixed + per_head_bytes(pl)) return PIVOT_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == PIVOT_BF16)
        return run_prefill<bf16_t>(pl, (const bf16_t *)q, (const bf16_t *)k, out_idx, out_score,
                                   (unsigned char *)workspace, workspace_bytes, st);
    return run_prefill<float>(pl, (const float *)q, (const float *)k, out_idx, out_score,
                              (unsigned char *)workspace, workspace_bytes, st);
}

int pivot_index_prefill(const void *q, const void *k, int32_t dtype, int64_t S, int32_t H, int32_t D,
                        int32_t top_k, int32_t g, double candidate_ratio, int32_t mode, int32_t *out_idx,
                        float *out_score, void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_common(q, k, dtype, S, H, D, top_k, g, candidate_ratio, mode, out_idx, out_score,
                          workspace, workspace_bytes, stream, false);
}

int dense_index(const void *q, const void *k, int32_t dtype, int64_t S, int32_t H, int32_t D, int32_t top_k,
                int32_t *out_idx, float *out_score, void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_common(q, k, dtype, S, H, D, top_k, 1, 1.0, PIVOT_REUSE, out_idx, out_score, workspace,
                          workspace_bytes, stream, true);
}

size_t pivot_decode_workspace_bytes(int32_t B, const int64_t *ctx_lens_host, int32_t g, int32_t H, int32_t D,
                                    int32_t top_k, double candidate_ratio, int32_t mode, int32_t dtype) {
    DecPlan dp;
    if (make_dec_plan(dp, B, ctx_lens_host, g, H, D, top_k, candidate_ratio, mode, dtype)) return 0;
    return dp.bytes;
}

int pivot_index_decode(const void *q, const void *k_cache, int32_t dtype, const int64_t *ctx_lens_host,
                       int32_t B, int32_t g, int32_t H, int32_t D, int32_t top_k, double candidate_ratio,
                       int32_t mode, int32_t *out_idx, float *out_score, void *workspace,
                       size_t workspace_bytes, void *stream) {
    DecPlan dp;
    int rc = make_dec_plan(dp, B, ctx_lens_host, g, H, D, top_k, candidate_ratio, mode, dtype);
    if (rc) return rc;
    if (!q || !k_cache || !out_idx) return PIVOT_EINVAL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned4(out_idx) || (out_score && !aligned4(out_score)))
        return PIVOT_EINVAL;
    if (!workspace || !aligned16(workspace) || workspace_bytes < dp.bytes) return PIVOT_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == PIVOT_BF16)
        return run_decode<bf16_t>(dp, ctx_lens_host, (const bf16_t *)q, (const bf16_t *)k_cache, out_idx,
                                  out_score, (unsigned char *)workspace, st);
    return run_decode<float>(dp, ctx_lens_host, (const float *)q, (const float *)k_cache, out_idx, out_score,
                             (unsigned char *)workspace, st);
}

int pivot_index_decode_noalloc(const void *q, const void *k_cache, int32_t dtype, const int64_t *ctx_lens_host,
                               int32_t B, int32_t g, int32_t H, int32_t D, int32_t top_k, double candidate_ratio,
                               int32_t mode, int32_t *out_idx, float *out_score, void *stream) {
    DecPlan dp;
    int rc = make_dec_plan(dp, B, ctx_lens_host, g, H, D, top_k, candidate_ratio, mode, dtype);
    if (rc) return rc;
    if (!q || !k_cache || !out_idx) return PIVOT_EINVAL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned4(out_idx) || (out_score && !aligned4(out_score)))
        return PIVOT_EINVAL;
    if (dp.bytes > STATIC_SCRATCH_BYTES) return PIVOT_EWORKSPACE;
    void *ws = nullptr;
    rc = static_scratch(&ws);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    t_prof_off = true;  // no event records: nothing is created during this call
    if (dtype == PIVOT_BF16)
        rc = run_decode<bf16_t>(dp, ctx_lens_host, (const bf16_t *)q, (const bf16_t *)k_cache, out_idx, out_score,
                                (unsigned char *)ws, st);
    else
        rc = run_decode<float>(dp, ctx_lens_host, (const float *)q, (const float *)k_cache, out_idx, out_score,
                               (unsigned char *)ws, st);
    t_prof_off = false;
    return rc;
}

int pivot_profile_enable(int on) {
    g_prof_on = on != 0;
    g_prof_used = 0;
    return PIVOT_OK;
}

int pivot_profile_read(double *ms_out, int64_t *count_out, int n_stages) {
    if (!ms_out || !count_out || n_stages < 0) return PIVOT_EINVAL;
    for (int i = 0; i < n_stages; ++i) {
        ms_out[i] = 0.0;
        count_out[i] = 0;
    }
    int rc = PIVOT_OK;
    for (int i = 0; i < g_prof_used; ++i) {
        const ProfRec &r = g_prof[i];
        float ms = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
            rc = PIVOT_EHIP;
            continue;
        }
        if (r.stage < n_stages) {
            ms_out[r.stage] += ms;
            count_out[r.stage] += 1;
        }
    }
    g_prof_used = 0;
    return rc;
}

}  // extern "C"
