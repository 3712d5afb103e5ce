// zs_kernels.hip -- the device side of libzeroshard.so for gfx950 (CDNA4):
// the fused multi-tensor Adam step, the N_d-slice gradient reduction, the
// reduction and the Adam step fused over a flat shard, and the gather of
// updated shards, each for fp16 or bfloat16 parameters and gradients; plus
// the plan upload and the launches behind the C ABI.
//
// All four kernels are elementwise HBM streams (Adam: 28 bytes per
// parameter; reduce: 2 N_d + 2 bytes; fused: 2 N_d + 26; gather: 4), so they
// use no matrix cores.  Every load and store instruction of a 64-lane wave
// covers one contiguous range (Adam: 512 bytes of fp16 or 1 KiB of fp32;
// reduce: 1 KiB of fp16; a parameter out of the other arrays' phase goes
// through a cross-lane permute into aligned 8-byte vectors), and streamed
// data moves with the nontemporal hint (the reduce's sparse output stream
// writes through L2 instead: st_through).
// On gfx950 nontemporal stores only stream at full rate when each
// instruction writes whole lines, which is why a lane's four-element groups
// of a wave tile are adjacent to its neighbours' (a 512-element tile
// interleaves two such groups across the wave instead of giving each lane
// eight neighbours), and why the gather aligns its tiles to the
// destination's 128-byte lines.
//
// Occupancy is capped on purpose.  The kernels run one 64-lane wave per
// workgroup, and each launch reserves dynamic LDS that the kernel never
// touches (the fused kernel uses 1 KiB of it), so that only a few workgroups
// are resident per CU (Adam 12 with 256-element tiles, 7 with 512-element
// tiles, 14-27 for lists of small tensors; reduce 4-16 on its 16- and
// 8-byte paths by slice count, 27 / 16 / 8 (28 / 16 / 12 on 8-byte groups)
// at 1 / 2 / 3 slices (32 elements per lane there); fused 5-12, twice that on its
// single-element path; gather 16).  Measured on MI355X, HBM3E streams these
// many-array patterns fastest with just enough bytes in flight to cover
// latency (about 45 KB per CU); with the 20-30 waves per CU that registers
// alone would allow, the same streams run 10-15% slower.  The Adam kernels
// are built for 7 waves per SIMD so that registers never cap below the 27
// workgroups per CU that plans of small tensors take.
//
// Exactness: every arithmetic step is one IEEE binary32 operation in a fixed
// order; the library is built with -ffp-contract=off (no fused multiply-add),
// fp32 denormals kept, and correctly rounded fp32 division and square root.
// fp16 <-> fp32 conversions are the hardware's (v_cvt_f32_f16 is exact,
// v_cvt_f16_f32 rounds to nearest even in the default mode).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>
#include <vector>

#include "zero_shard.h"
#include "zs_internal.h"

namespace {

using zs::Chunk;
using zs::kAdamTileFine;
using zs::kTile;
using zs::kWave;
using zs::TensorDesc;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// The 16-bit formats of parameters and gradients: IEEE binary16 (the
// pages' ledger) and bfloat16 (the variant that keeps the same ledger with
// bfloat16 in their place).  Widening is exact in both; narrowing rounds
// to nearest even (v_cvt_f16_f32, v_cvt_pk_bf16_f32).  A value is infinite
// or NaN when its exponent field is all ones.
struct FmtF16 {
    typedef _Float16 T;
    typedef f16x4 V4;
    typedef f16x8 V8;
    static constexpr uint16_t kExp = 0x7C00;
};
struct FmtBF16 {
    typedef __bf16 T;
    typedef bf16x4 V4;
    typedef bf16x8 V8;
    static constexpr uint16_t kExp = 0x7F80;
};

// Pointers read from the chunk table are generic; the arrays live in device
// global memory, and saying so lets the compiler use global_load/store
// instead of flat accesses.
#define ZS_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ ZS_GLOBAL T *as_global(T *p) {
    return (ZS_GLOBAL T *)p;
}
template <typename T>
__device__ __forceinline__ const ZS_GLOBAL T *as_global(const T *p) {
    return (const ZS_GLOBAL T *)p;
}

struct AdamConsts {
    float lr, b1, omb1, b2, omb2, bc1, bc2, eps;
    float unscale; // 2^-k for gradients that carry a loss scale 2^k, else 1
};

template <typename T>
__device__ __forceinline__ T ld_nt(const T *p) {
    return __builtin_nontemporal_load(as_global(p));
}
template <typename T>
__device__ __forceinline__ void st_nt(T v, T *p) {
    __builtin_nontemporal_store(v, as_global(p));
}

// A store that writes through L2 at system scope (cache policy sc0 sc1) for
// 8- or 16-byte vectors.  For the reduce's output, a sparse write stream
// (2 bytes per element against 2 N_d read), it ran 1.5% (N_d = 64) to 4%
// (N_d = 4, 8) faster than nontemporal stores on MI355X, interleaved in one
// process on two boxes, with identical results; on the write-heavy Adam
// step and gather it was 4-6% slower, so those keep nontemporal stores.
// No builtin sets these cache-policy bits on a global store; the asm has
// no outputs, and a store the compiler does not count only makes its
// later waits on the memory counter stricter.
template <typename V>
__device__ __forceinline__ void st_through(V v, V *p) {
    static_assert(sizeof(V) == 16 || sizeof(V) == 8, "8- or 16-byte vectors");
    if constexpr (sizeof(V) == 16)
        asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
    else
        asm volatile("global_store_dwordx2 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}

template <class Fmt = FmtF16>
__device__ __forceinline__ bool bits_nonfinite(uint16_t b) {
    return (b & Fmt::kExp) == Fmt::kExp;
}

// Raise the non-finite flag once for this wave if any lane saw a non-finite
// value.  The flag only ever goes from 0 to 1, so a wave that reads 1 (an
// agent-coherent load) skips its atomic: with many waves seeing infinities
// only the first few reach the flag's address.
__device__ __forceinline__ void raise_flag(int32_t *flag, int bad) {
    if (flag == nullptr)
        return;
    if (__ballot(bad) != 0 && threadIdx.x % 64u == 0) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
            __hip_atomic_fetch_or(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// Adam step.
// ---------------------------------------------------------------------------

// One element of the Adam step (Kingma and Ba, Algorithm 1, with bias
// correction and eps outside the root).  Returns the new 16-bit parameter;
// `bad` is raised if the gradient the update uses, after the loss scale's
// 2^-k, is infinite or NaN.  The product is exact for every finite fp16
// value; a finite bfloat16 value (fp32's exponent range) can underflow for
// k > 0 and overflow to infinity for k < 0, which the flag then reports.
template <class Fmt = FmtF16>
__device__ __forceinline__ typename Fmt::T adam_elem(float g, float &w, float &m, float &v,
                                                     const AdamConsts &c, int &bad) {
    g = g * c.unscale;
    bad |= (__float_as_uint(g) & 0x7F800000u) == 0x7F800000u;
    const float m_old = c.b1 * m;
    const float m_in = c.omb1 * g;
    m = m_old + m_in;
    const float v_old = c.b2 * v;
    const float g2 = g * g;
    const float v_in = c.omb2 * g2;
    v = v_old + v_in;
    const float m_hat = m / c.bc1;
    const float v_hat = v / c.bc2;
    const float denom = __builtin_sqrtf(v_hat) + c.eps;
    const float u = m_hat / denom;
    const float step = c.lr * u;
    w = w - step;
    return (typename Fmt::T)w;
}

template <class Fmt>
__device__ __forceinline__ void adam_single(const TensorDesc &T, uint64_t i,
                                            const AdamConsts &c, int &bad) {
    const uint16_t gb = as_global(T.g)[i];
    typename Fmt::T gh;
    memcpy(&gh, &gb, 2);
    float w = as_global(T.w)[i], m = as_global(T.m)[i], v = as_global(T.v)[i];
    const typename Fmt::T p = adam_elem<Fmt>((float)gh, w, m, v, c, bad);
    as_global(T.w)[i] = w;
    as_global(T.m)[i] = m;
    as_global(T.v)[i] = v;
    uint16_t pb;
    memcpy(&pb, &p, 2);
    as_global(T.p)[i] = pb;
}

// Four consecutive elements held in registers: fp16 gradient (8 bytes) and
// fp32 master, m, v (16 bytes each).
template <class Fmt>
struct Quad {
    typename Fmt::V4 g;
    f32x4 w, m, v;
};

template <class Fmt>
__device__ __forceinline__ void quad_load(const TensorDesc &T, uint64_t i, Quad<Fmt> &q) {
    q.g = ld_nt(reinterpret_cast<const typename Fmt::V4 *>(T.g + i));
    q.w = ld_nt(reinterpret_cast<const f32x4 *>(T.w + i));
    q.m = ld_nt(reinterpret_cast<const f32x4 *>(T.m + i));
    q.v = ld_nt(reinterpret_cast<const f32x4 *>(T.v + i));
}

// The update of four elements held in registers; stores the fp32 state and
// returns the new parameter.
template <class Fmt>
__device__ __forceinline__ typename Fmt::V4 quad_update(const TensorDesc &T, uint64_t i,
                                                        Quad<Fmt> &q, const AdamConsts &c,
                                                        int &bad) {
    typename Fmt::V4 p;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const typename Fmt::T gj = q.g[j];
        float w = q.w[j], m = q.m[j], v = q.v[j];
        p[j] = adam_elem<Fmt>((float)gj, w, m, v, c, bad);
        q.w[j] = w;
        q.m[j] = m;
        q.v[j] = v;
    }
    st_nt(q.w, reinterpret_cast<f32x4 *>(T.w + i));
    st_nt(q.m, reinterpret_cast<f32x4 *>(T.m + i));
    st_nt(q.v, reinterpret_cast<f32x4 *>(T.v + i));
    return p;
}

// Stores of a 16-bit output (the parameter; the fused step's gradient
// output too) that is s elements (1-3) out of the phase of the arrays its
// values come from.  Lane L holds the new values of elements 4L..4L+3 of a
// run from the vector-aligned element `base`; the output's 8-byte vectors
// start at elements 4L - s.  Lane L >= 1 joins the last s values of lane
// L - 1 (a cross-lane permute) with its own first 4 - s and stores one
// aligned vector; the run's first 4 - s and last s elements, whose vectors
// the neighbouring elements share, go singly.  Every byte written belongs
// to the run's own elements.

// The vector that starts s elements before this lane's group: the last s
// values of `src` as lane L - 1 holds it, then the first 4 - s of `own`.
__device__ __forceinline__ uint64_t join_shifted(uint64_t own, uint64_t src, uint32_t lane,
                                                 uint32_t s) {
    const int from = (int)(((lane + kWave - 1u) % kWave) * 4u); // lane 0's is unused
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)(uint32_t)src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)(uint32_t)(src >> 32));
    const uint64_t prev = ((uint64_t)hi << 32) | lo;
    return (prev >> (16u * (4u - s))) | (own << (16u * s));
}

// The run's edges: the first 4 - s values of lane 0's group and the last s
// of lane `last_lane`'s (`vals`: this lane's group, at element `at`).
__device__ __forceinline__ void store_edges(uint16_t *dst, uint32_t lane, uint32_t s,
                                            uint32_t last_lane, uint64_t vals, uint64_t at) {
    uint16_t b[4];
    memcpy(b, &vals, 8);
#pragma unroll
    for (uint32_t j = 0; j < 4; j++)
        if (j < 4u - s ? lane == 0 : lane == last_lane)
            st_nt(b[j], dst + at + j);
}

// nq <= 64 groups held by lanes 0..nq-1 (exactly these lanes take part): a
// tensor's head or the groups of a partial tile.  V: the 8-byte vector of
// four 16-bit values.
template <typename V>
__device__ __forceinline__ void shifted_store_groups(uint16_t *dst, uint32_t s, uint64_t base,
                                                     uint32_t lane, uint32_t nq, V p) {
    static_assert(sizeof(V) == 8, "four 16-bit values");
    uint64_t own;
    memcpy(&own, &p, 8);
    const uint64_t joined = join_shifted(own, own, lane, s);
    if (lane != 0)
        st_nt(joined, reinterpret_cast<uint64_t *>(dst + base + 4u * lane - s));
    store_edges(dst, lane, s, nq - 1u, own, base + 4u * lane);
}

// A full tile of Q runs of 256 (lane L: elements 4L..4L+3 of each run from
// `base`): lane 0 of run k >= 1 joins the last s values of run k - 1,
// which lane 63 hands it through the same permute, and stores a whole
// vector, so that only the tile's first 4 - s and last s elements go
// singly.
template <typename V, int Q>
__device__ __forceinline__ void shifted_store_tile(uint16_t *dst, uint32_t s, uint64_t base,
                                                   uint32_t lane, const V (&p)[Q]) {
    static_assert(sizeof(V) == 8, "four 16-bit values");
    uint64_t own[Q];
    memcpy(own, p, sizeof(own));
#pragma unroll
    for (int k = 0; k < Q; k++) {
        const uint64_t src = k > 0 && lane == kWave - 1u ? own[(k + Q - 1) % Q] : own[k];
        const uint64_t joined = join_shifted(own[k], src, lane, s);
        if (k > 0 || lane != 0)
            st_nt(joined, reinterpret_cast<uint64_t *>(dst + base + 4u * kWave * k +
                                                       4u * lane - s));
    }
    const bool first = lane == 0;
    store_edges(dst, lane, s, kWave - 1u, first ? own[0] : own[Q - 1],
                base + (first ? 0u : 4u * kWave * (Q - 1)) + 4u * lane);
}

// The four values of a 16-bit input that is s elements (1-3) out of phase
// at element i (vector-aligned for the other arrays): they lie in the two
// aligned 8-byte words from element i - s, which every lane loads whole and
// joins in registers, with no cross-lane step and no lane conditions.  The
// words also hold s elements before i and 4 - s after i + 3, which are
// discarded; an aligned word holding an element of the array lies in a
// page that holds the array's own bytes, so reading it cannot fault, and
// a neighbouring tile that writes those elements meanwhile (the gradient
// read from the parameter's place) changes only discarded values.
__device__ __forceinline__ uint64_t load_shifted(const uint16_t *src, uint32_t s, uint64_t i) {
    const uint64_t *word = reinterpret_cast<const uint64_t *>(src + i - s);
    const uint64_t lo = ld_nt(word), hi = ld_nt(word + 1);
    return (lo >> (16u * s)) | (hi << (16u * (4u - s)));
}

// The Adam step's access modes on the vector path, decided once per tile
// so that each mode's code is what it would be without the others:
// kInPhase, every array in phase; kParamShift, the parameter s = T.pshift
// out of phase (shifted stores); kGradShift, the gradient T.gshift out of
// phase (shifted loads) and the parameter in phase or out by T.pshift.
enum { kInPhase = 0, kParamShift = 1, kGradShift = 2 };

// The parameter stores of nq <= 64 groups held by lanes 0..nq-1 (only
// these lanes take part).
template <class Fmt, int MODE>
__device__ __forceinline__ void param_store_quads(const TensorDesc &T, uint64_t base,
                                                  uint32_t lane, uint32_t nq,
                                                  typename Fmt::V4 p) {
    if (MODE == kInPhase || (MODE == kGradShift && T.pshift == 0))
        st_nt(p, reinterpret_cast<typename Fmt::V4 *>(T.p + base + 4u * lane));
    else
        shifted_store_groups(T.p, T.pshift, base, lane, nq, p);
}

// The four elements from i into q: the fp32 state, and the gradient
// shifted or not.
template <class Fmt, int MODE>
__device__ __forceinline__ void quad_load_mode(const TensorDesc &T, uint64_t i, Quad<Fmt> &q) {
    if constexpr (MODE == kGradShift) {
        q.w = ld_nt(reinterpret_cast<const f32x4 *>(T.w + i));
        q.m = ld_nt(reinterpret_cast<const f32x4 *>(T.m + i));
        q.v = ld_nt(reinterpret_cast<const f32x4 *>(T.v + i));
        const uint64_t g = load_shifted(T.g, T.gshift, i);
        memcpy(&q.g, &g, 8);
    } else {
        quad_load<Fmt>(T, i, q);
    }
}

// count (65..64 G) consecutive elements from `lo` in one pass over memory,
// whatever the arrays' phases: lane L takes elements L + 64k, k < G, every
// lane loading all G of its elements first (an index past the end clamped
// to the last element, so that no load waits on a lane condition and the
// wave waits on memory once), then updating and storing those in range.
// In the 512-element kernel it takes a tensor's partial last tile, or a
// whole small chunk, of more than 64 elements, which the head / groups /
// singles sequence covered in two or three passes.  Measured on MI355X against that sequence (one
// process, identical outputs, fraction of 8 TB/s): lists of 300- and
// 1,000-element tensors 0.56 and 0.75 against 0.48 and 0.60, random sizes
// 1-1,024 0.70 against 0.57 and 1-8,192 0.70 against 0.65; at 64
// elements or fewer, where the sequence is one pass, the span's seven
// extra loads per lane and array lost (0.36 against 0.38-0.44), so those
// keep it.
template <class Fmt, int G>
__device__ __forceinline__ void adam_span_g(const TensorDesc &T, uint64_t lo, uint32_t count,
                                            const AdamConsts &c, int &bad) {
    const uint32_t lane = threadIdx.x;
    uint16_t gb[G];
    float w[G], m[G], v[G];
#pragma unroll
    for (int k = 0; k < G; k++) {
        const uint64_t i = lo + min(lane + kWave * k, count - 1u);
        gb[k] = as_global(T.g)[i];
        w[k] = as_global(T.w)[i];
        m[k] = as_global(T.m)[i];
        v[k] = as_global(T.v)[i];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < G; k++) {
        if (lane + kWave * k >= count)
            continue;
        const uint64_t i = lo + lane + kWave * k;
        typename Fmt::T gh;
        memcpy(&gh, &gb[k], 2);
        const typename Fmt::T p = adam_elem<Fmt>((float)gh, w[k], m[k], v[k], c, bad);
        as_global(T.w)[i] = w[k];
        as_global(T.m)[i] = m[k];
        as_global(T.v)[i] = v[k];
        uint16_t pb;
        memcpy(&pb, &p, 2);
        as_global(T.p)[i] = pb;
    }
}

// A full Adam tile: TILE consecutive elements from `base` (vector-aligned),
// TILE / 256 groups of four per lane.  Lane L takes elements 4L..4L+3 of
// every 256, so each of the wave's load and store instructions covers one
// contiguous 512-byte (16-bit) or 1-KiB (fp32) range (a shifted 16-bit
// array's: 504 or 512 bytes, plus a shifted store's edges).  All loads are
// issued before any arithmetic.
template <class Fmt, uint32_t TILE, int MODE>
__device__ __forceinline__ void adam_tile(const TensorDesc &T, uint64_t base, uint32_t lane,
                                          const AdamConsts &c, int &bad) {
    constexpr int Q = TILE / (4 * kWave);
    static_assert(Q * 4 * kWave == TILE, "whole groups of four per lane");
    Quad<Fmt> a[Q];
#pragma unroll
    for (int k = 0; k < Q; k++)
        quad_load_mode<Fmt, MODE>(T, base + 4u * lane + 4u * kWave * k, a[k]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MODE == kInPhase) {
#pragma unroll
        for (int k = 0; k < Q; k++) {
            const uint64_t i = base + 4u * lane + 4u * kWave * k;
            st_nt(quad_update<Fmt>(T, i, a[k], c, bad),
                  reinterpret_cast<typename Fmt::V4 *>(T.p + i));
        }
    } else {
        typename Fmt::V4 p[Q];
#pragma unroll
        for (int k = 0; k < Q; k++)
            p[k] = quad_update<Fmt>(T, base + 4u * lane + 4u * kWave * k, a[k], c, bad);
        if (MODE == kGradShift && T.pshift == 0) {
#pragma unroll
            for (int k = 0; k < Q; k++)
                st_nt(p[k], reinterpret_cast<typename Fmt::V4 *>(T.p + base + 4u * lane +
                                                                  4u * kWave * k));
        } else {
            shifted_store_tile(T.p, T.pshift, base, lane, p);
        }
    }
}

// nq <= 64 groups of four from the vector-aligned element `base`, held by
// lanes 0..nq-1 (only these lanes take part): a head's or a partial tile's.
template <class Fmt, int MODE>
__device__ __forceinline__ void adam_quads(const TensorDesc &T, uint64_t base, uint32_t lane,
                                           uint32_t nq, const AdamConsts &c, int &bad) {
    Quad<Fmt> x;
    quad_load_mode<Fmt, MODE>(T, base + 4u * lane, x);
    param_store_quads<Fmt, MODE>(T, base, lane, nq, quad_update<Fmt>(T, base + 4u * lane, x, c,
                                                                       bad));
}

// The peeled head of a tensor on the vector path: its first `count`
// elements (count <= T.head < 256).  The first T.head % 4 go singly (they
// precede the first aligned vector), then at most 63 groups of four, one per
// lane; a tensor that ends inside its head does its last fewer-than-four
// singly.
template <class Fmt, int MODE>
__device__ __forceinline__ void adam_head(const TensorDesc &T, uint32_t count,
                                          const AdamConsts &c, int &bad) {
    const uint32_t lane = threadIdx.x;
    const uint32_t singles = min(T.head % 4u, count);
    if (lane < singles)
        adam_single<Fmt>(T, lane, c, bad);
    const uint32_t nquads = (count - singles) / 4u;
    if (lane < nquads)
        adam_quads<Fmt, MODE>(T, singles, lane, nquads, c, bad);
    const uint32_t rest = count - singles - 4u * nquads;
    if (lane < rest)
        adam_single<Fmt>(T, singles + 4u * nquads + lane, c, bad);
}

// Tile j of a chunk on the vector path.  The tensor's peeled head (up to
// where its fp32 arrays reach a 1 KiB boundary on tensors of 1,024 elements
// or more, else only to the first aligned vector) rides in its first chunk
// and is done by tile 0; every other chunk starts at the head plus a whole
// number of tiles.  The chunk's last, partial tile goes four elements per
// lane, then the final fewer-than-four singly.  MODE: which 16-bit array
// is out of phase (kInPhase, kParamShift, kGradShift).
template <class Fmt, uint32_t TILE, int MODE>
__device__ __forceinline__ void adam_tile_of_chunk(const TensorDesc &T, const Chunk &ch,
                                                   uint32_t j, const AdamConsts &c, int &bad) {
    const uint32_t lane = threadIdx.x;
    // one-pass spans in the 512-element kernel, which plans of small
    // tensors take; the 256-element kernel (big tensors, one partial tile
    // each) keeps the former sequence (with the spans compiled in, big
    // plans ran 0.2% slower)
    constexpr bool kSpans = TILE == kTile;
    if (kSpans && ch.count < TILE && ch.count > kWave) {
        // the whole chunk (a small tensor, its head included) in one pass:
        // whole groups of four, one per lane, when it is just that (in
        // phase, from a vector-aligned start, at most 64 groups), else
        // element by element
        if (j != 0)
            return;
        const uint32_t head = ch.start == 0 ? T.head : 0u;
        if (MODE == kInPhase && head == 0 && ch.count % 4u == 0 && ch.count <= 4u * kWave) {
            if (lane < ch.count / 4u)
                adam_quads<Fmt, kInPhase>(T, ch.start, lane, ch.count / 4u, c, bad);
        } else {
            adam_span_g<Fmt, TILE / kWave>(T, ch.start, ch.count, c, bad);
        }
        return;
    }
    const uint32_t head = ch.start == 0 ? min(T.head, ch.count) : 0u;
    if (j == 0 && head != 0)
        adam_head<Fmt, MODE>(T, head, c, bad);
    const uint64_t base = ch.start + head;
    const uint32_t body = ch.count - head;
    const uint32_t nfull = body / TILE;
    if (j < nfull) {
        adam_tile<Fmt, TILE, MODE>(T, base + (uint64_t)j * TILE, lane, c, bad);
        return;
    }
    if (j > nfull)
        return; // past the end of a short chunk
    const uint64_t rbase = base + (uint64_t)nfull * TILE;
    const uint32_t rem = body - nfull * TILE; // < TILE
    if (kSpans && rem > kWave) {
        adam_span_g<Fmt, TILE / kWave>(T, rbase, rem, c, bad);
        return;
    }
    // groups of four, one per lane (in rounds of 64), then singly
    const uint32_t nquads = rem / 4u;
    if constexpr (MODE != kInPhase) {
        for (uint32_t r0 = 0; r0 < nquads; r0 += kWave) {
            const uint32_t nq = min(nquads - r0, kWave);
            if (lane < nq)
                adam_quads<Fmt, MODE>(T, rbase + 4u * r0, lane, nq, c, bad);
        }
    } else {
        for (uint32_t q = lane; q < nquads; q += kWave) {
            Quad<Fmt> x;
            const uint64_t i = rbase + 4u * q;
            quad_load<Fmt>(T, i, x);
            st_nt(quad_update<Fmt>(T, i, x, c, bad), reinterpret_cast<typename Fmt::V4 *>(T.p + i));
        }
    }
    const uint32_t tail = rem - 4u * nquads;
    if (lane < tail)
        adam_single<Fmt>(T, rbase + 4u * nquads + lane, c, bad);
}

// Tile j of a chunk on the vector path in the tensor's mode.
template <class Fmt, uint32_t TILE>
__device__ __forceinline__ void adam_tile_vec(const TensorDesc &T, const Chunk &ch, uint32_t j,
                                              const AdamConsts &c, int &bad) {
    if ((T.pshift | T.gshift) == 0)
        adam_tile_of_chunk<Fmt, TILE, kInPhase>(T, ch, j, c, bad);
    else if (T.gshift == 0)
        adam_tile_of_chunk<Fmt, TILE, kParamShift>(T, ch, j, c, bad);
    else
        adam_tile_of_chunk<Fmt, TILE, kGradShift>(T, ch, j, c, bad);
}

// Tile j of a chunk of a tensor whose arrays disagree in alignment: single
// elements, lane-strided so each access instruction of the wave stays
// contiguous.  A full tile loads all of a lane's TILE / 64 elements before
// the first update (the same per-element operations as adam_single), so
// the wave keeps as many loads in flight as on the vector path; a partial
// tile goes element by element.
template <class Fmt, uint32_t TILE>
__device__ __forceinline__ void adam_tile_single(const TensorDesc &T, const Chunk &ch,
                                                 uint32_t j, const AdamConsts &c, int &bad) {
    const uint32_t lo = j * TILE;
    if (lo >= ch.count)
        return; // past the end of a short chunk
    const uint32_t hi = min(ch.count, lo + TILE);
    if (hi - lo == TILE) {
        constexpr int G = TILE / kWave;
        const uint64_t i0 = ch.start + lo + threadIdx.x;
        uint16_t gb[G];
        float w[G], m[G], v[G];
#pragma unroll
        for (int k = 0; k < G; k++) {
            const uint64_t i = i0 + (uint64_t)kWave * k;
            gb[k] = as_global(T.g)[i];
            w[k] = as_global(T.w)[i];
            m[k] = as_global(T.m)[i];
            v[k] = as_global(T.v)[i];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < G; k++) {
            const uint64_t i = i0 + (uint64_t)kWave * k;
            typename Fmt::T gh;
            memcpy(&gh, &gb[k], 2);
            const typename Fmt::T p = adam_elem<Fmt>((float)gh, w[k], m[k], v[k], c, bad);
            as_global(T.w)[i] = w[k];
            as_global(T.m)[i] = m[k];
            as_global(T.v)[i] = v[k];
            uint16_t pb;
            memcpy(&pb, &p, 2);
            as_global(T.p)[i] = pb;
        }
        return;
    }
    if (TILE == kTile && hi - lo > kWave) {
        adam_span_g<Fmt, TILE / kWave>(T, ch.start + lo, hi - lo, c, bad);
        return;
    }
    for (uint32_t k = lo + threadIdx.x; k < hi; k += kWave)
        adam_single<Fmt>(T, ch.start + k, c, bad);
}

// The fused step over a plan.  Each workgroup is one wave and takes one Adam
// tile: virtual workgroup b is tile b % tiles_per_chunk of chunk
// b / tiles_per_chunk.  Launches with fewer workgroups than virtual ones
// stride over them.  Fmt: the 16-bit format of parameters and gradients;
// TILE: the plan's Adam tile (kAdamTileFine or kTile elements).
template <class Fmt, uint32_t TILE, bool SHIFTS>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(7))) void zs_adam_kernel(
    const TensorDesc *__restrict__ tensors, const Chunk *__restrict__ chunks,
    uint64_t n_virtual, uint32_t tiles_per_chunk, AdamConsts c, int32_t *__restrict__ flag,
    const int32_t *__restrict__ skip, const int32_t *__restrict__ log2_scale) {
    if (skip != nullptr && *skip != 0)
        return; // the same value for every wave: the whole step is skipped
    if (log2_scale != nullptr) {
        const int k = min(max(*log2_scale, -ZERO_LOG2_SCALE_MAX), ZERO_LOG2_SCALE_MAX);
        c.unscale = __uint_as_float((uint32_t)(127 - k) << 23); // 2^-k, a normal fp32
    }
    int bad = 0;
    for (uint64_t vb = blockIdx.x; vb < n_virtual; vb += gridDim.x) {
        const uint64_t ci = vb / tiles_per_chunk;
        const uint32_t j = (uint32_t)(vb - ci * tiles_per_chunk);
        const Chunk ch = chunks[ci];
        const TensorDesc T = tensors[ch.tensor];
        if (T.vec == 4) {
            if constexpr (SHIFTS)
                adam_tile_vec<Fmt, TILE>(T, ch, j, c, bad);
            else
                adam_tile_of_chunk<Fmt, TILE, kInPhase>(T, ch, j, c, bad);
        } else {
            adam_tile_single<Fmt, TILE>(T, ch, j, c, bad);
        }
    }
    raise_flag(flag, bad);
}

// The Adam step over one tensor whose descriptor travels by value (no
// table): workgroup b takes tile b of the tensor, which stands in for a
// chunk of one tile (tile 0 also holds the peeled head), so the per-tile
// code, and the results, are those of zs_adam_kernel.  Used where no table
// exists: the second half of zero_reduce_adam_step at many slices.
// The host gives the element counts of the first and the last tile; the
// kernel picks a tile's count with equality tests only.  (A count taken as
// min(n - start, TILE) on the device was miscompiled by this toolchain for
// the single-element path: a VALU 64-bit compare feeding a scalar select
// that read a stale SCC, so every partial tile ran as a full one.)
template <class Fmt, uint32_t TILE, bool SHIFTS>
__global__ __launch_bounds__(kWave) void zs_adam_flat_kernel(TensorDesc T, uint64_t ntiles,
                                                             uint32_t first_count,
                                                             uint32_t last_count, AdamConsts c,
                                                             int32_t *__restrict__ flag) {
    int bad = 0;
    const uint64_t h = T.vec == 4 && T.head < T.n ? T.head : 0;
    for (uint64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        Chunk ch;
        ch.tensor = 0;
        ch.start = b == 0 ? 0 : h + b * TILE;
        ch.count = b == ntiles - 1 ? last_count : (b == 0 ? first_count : TILE);
        if (T.vec == 4) {
            if constexpr (SHIFTS)
                adam_tile_vec<Fmt, TILE>(T, ch, 0, c, bad);
            else
                adam_tile_of_chunk<Fmt, TILE, kInPhase>(T, ch, 0, c, bad);
        } else {
            adam_tile_single<Fmt, TILE>(T, ch, 0, c, bad);
        }
    }
    raise_flag(flag, bad);
}

// ---------------------------------------------------------------------------
// Gradient reduction over N_d slices.
// ---------------------------------------------------------------------------
struct SliceArgs {
    const uint16_t *p[ZERO_MAX_SLICES]; // 16-bit values of the kernel's format
};

// Vector of VEC values of a format.
template <class Fmt, int VEC>
struct HVec;
template <class Fmt>
struct HVec<Fmt, 8> {
    typedef typename Fmt::V8 T;
};
template <class Fmt>
struct HVec<Fmt, 4> {
    typedef typename Fmt::V4 T;
};

template <class Fmt = FmtF16>
__device__ __forceinline__ float widen(const uint16_t *p, uint64_t i) {
    return (float)as_global(reinterpret_cast<const typename Fmt::T *>(p))[i];
}

template <class Fmt = FmtF16>
__device__ __forceinline__ float reduce_single(const SliceArgs &s, uint32_t nd, uint64_t i) {
    float acc = widen<Fmt>(s.p[0], i);
    for (uint32_t r = 1; r < nd; r++)
        acc = acc + widen<Fmt>(s.p[r], i);
    return acc;
}

// Adds slices r0 .. r0+B-1, in rank order, at group start i into acc; the B
// loads are all issued before the first add.  With `first`, slice r0
// initialises the sum instead of being added to it.
template <int VEC, int B, class Fmt = FmtF16>
__device__ __forceinline__ void reduce_batch(const SliceArgs &s, uint32_t r0, uint64_t i,
                                             bool first, float (&acc)[VEC]) {
    typedef typename HVec<Fmt, VEC>::T hv;
    hv x[B];
#pragma unroll
    for (int q = 0; q < B; q++)
        x[q] = ld_nt(reinterpret_cast<const hv *>(s.p[r0 + q] + i));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < B; q++)
#pragma unroll
        for (int j = 0; j < VEC; j++)
            acc[j] = (first && q == 0) ? (float)x[0][j] : acc[j] + (float)x[q][j];
}

// Slices r0 .. r0+rest-1 (rest = 1-15) as one batch: every load in flight
// before the first add.
template <int VEC, class Fmt>
__device__ __forceinline__ void reduce_rest(const SliceArgs &s, uint32_t r0, uint32_t rest,
                                            uint64_t i, float (&acc)[VEC]) {
    const bool first = r0 == 0;
    switch (rest) {
#define ZS_REST(R)                                                                                 \
    case R:                                                                                        \
        reduce_batch<VEC, R, Fmt>(s, r0, i, first, acc);                                          \
        break;
        ZS_REST(1) ZS_REST(2) ZS_REST(3) ZS_REST(4) ZS_REST(5) ZS_REST(6) ZS_REST(7) ZS_REST(8)
        ZS_REST(9) ZS_REST(10) ZS_REST(11) ZS_REST(12) ZS_REST(13) ZS_REST(14) ZS_REST(15)
#undef ZS_REST
    default:
        break;
    }
}

// One vector group of VEC outputs at element i: the sum over the nd slices
// in rank order, then one division by nd.  VEC = 8: batches of 16 slices in
// flight per lane, then the rest in one batch; VEC = 4: batches of 16, 8, 4
// and 1.
template <class Fmt, int VEC>
__device__ __forceinline__ typename HVec<Fmt, VEC>::T reduce_group_value(const SliceArgs &s,
                                                                        uint32_t nd, uint64_t i,
                                                                        float count, int &bad) {
    typedef typename HVec<Fmt, VEC>::T hv;
    float acc[VEC];
    uint32_t r = 0;
    for (; r + 16 <= nd; r += 16)
        reduce_batch<VEC, 16, Fmt>(s, r, i, r == 0, acc);
    if constexpr (VEC == 8) {
        if (r < nd)
            reduce_rest<VEC, Fmt>(s, r, nd - r, i, acc);
    } else {
        for (; r + 8 <= nd; r += 8)
            reduce_batch<VEC, 8, Fmt>(s, r, i, r == 0, acc);
        for (; r + 4 <= nd; r += 4)
            reduce_batch<VEC, 4, Fmt>(s, r, i, r == 0, acc);
        for (; r < nd; r++)
            reduce_batch<VEC, 1, Fmt>(s, r, i, r == 0, acc);
    }
    hv o;
#pragma unroll
    for (int j = 0; j < VEC; j++) {
        o[j] = (typename Fmt::T)(acc[j] / count);
        uint16_t b;
        typename Fmt::T oj = o[j];
        memcpy(&b, &oj, 2);
        bad |= bits_nonfinite<Fmt>(b);
    }
    return o;
}

// The same, stored at out + i.
template <class Fmt, int VEC>
__device__ __forceinline__ void reduce_group(const SliceArgs &s, uint32_t nd, uint64_t i,
                                             float count, uint16_t *out, int &bad) {
    typedef typename HVec<Fmt, VEC>::T hv;
    st_through(reduce_group_value<Fmt, VEC>(s, nd, i, count, bad), reinterpret_cast<hv *>(out + i));
}

// The reduce's output of nq <= 64 groups of eight held by lanes 0..nq-1
// (lane L: elements 8L..8L+7 from `base`, exactly these lanes take part)
// when the output is s elements (1-3) out of the slices' phase: lane L
// stores the aligned vector of its elements 4 - s..7 - s whole, and the
// one before it joined with the last s values of lane L - 1 (a cross-lane
// permute); the first 4 - s and the last s elements go singly.
template <typename V8>
__device__ __forceinline__ void reduce_store_shifted8(uint16_t *out, uint32_t s, uint64_t base,
                                                      uint32_t lane, uint32_t nq, V8 o) {
    static_assert(sizeof(V8) == 16, "eight 16-bit values");
    uint64_t h[2];
    memcpy(h, &o, 16);
    const uint64_t at = base + 8u * lane;
    st_through((h[0] >> (16u * (4u - s))) | (h[1] << (16u * s)),
               reinterpret_cast<uint64_t *>(out + at + 4u - s));
    const uint64_t joined = join_shifted(h[0], h[1], lane, s);
    if (lane != 0)
        st_through(joined, reinterpret_cast<uint64_t *>(out + at - s));
    uint16_t b[8];
    memcpy(b, &o, 16);
#pragma unroll
    for (uint32_t j = 0; j < 4; j++) {
        if (lane == 0 && j < 4u - s)
            as_global(out)[at + j] = b[j];
        if (lane == nq - 1u && j >= 4u - s)
            as_global(out)[at + 4u + j] = b[4 + j];
    }
}

template <class Fmt>
__device__ __forceinline__ void reduce_one(const SliceArgs &s, uint32_t nd, uint64_t i,
                                           float count, uint16_t *out, int &bad) {
    const typename Fmt::T o = (typename Fmt::T)(reduce_single<Fmt>(s, nd, i) / count);
    uint16_t b;
    memcpy(&b, &o, 2);
    as_global(out)[i] = b;
    bad |= bits_nonfinite<Fmt>(b);
}

// Each lane reduces one vector group of VEC elements (grid-striding when the
// launch is smaller than the work); the unaligned head (fewer than VEC
// leading elements) and the tail past the last whole group go one element
// per lane.  VEC = 1: every element singly.  SHIFT (VEC = 8): the output
// is oshift elements out of the slices' phase and each wave's 64 groups
// are stored shifted.
template <class Fmt, int VEC, bool SHIFT = false>
__global__ __launch_bounds__(kWave) void zs_reduce_kernel(SliceArgs s, uint32_t nd, uint64_t n,
                                                          uint32_t head, uint16_t *__restrict__ out,
                                                          int32_t *__restrict__ flag,
                                                          uint32_t oshift) {
    const float count = (float)nd;
    const uint64_t gtid = (uint64_t)blockIdx.x * kWave + threadIdx.x;
    const uint64_t gstride = (uint64_t)gridDim.x * kWave;
    int bad = 0;
    const uint64_t h = head < n ? head : n;
    const uint64_t ngroups = VEC > 1 ? (n - h) / VEC : 0;
    const uint64_t body_end = h + ngroups * VEC;
    if (gtid < h)
        reduce_one<Fmt>(s, nd, gtid, count, out, bad);
    for (uint64_t i = body_end + gtid; i < n; i += gstride)
        reduce_one<Fmt>(s, nd, i, count, out, bad);
    if constexpr (SHIFT) {
        static_assert(VEC == 8, "shifted output on the 16-byte path");
        const uint32_t lane = threadIdx.x;
        for (uint64_t k0 = (uint64_t)blockIdx.x * kWave; k0 < ngroups; k0 += gstride) {
            const uint32_t nq = (uint32_t)min(ngroups - k0, (uint64_t)kWave);
            if (lane < nq)
                reduce_store_shifted8(out, oshift, h + k0 * 8u, lane, nq,
                                      reduce_group_value<Fmt, 8>(s, nd, h + (k0 + lane) * 8u,
                                                                 count, bad));
        }
    } else if (VEC > 1) {
        for (uint64_t k = gtid; k < ngroups; k += gstride)
            reduce_group<Fmt, VEC == 8 ? 8 : 4>(s, nd, h + k * VEC, count, out, bad);
    }
    raise_flag(flag, bad);
}

// The reduction over ND = 1-3 slices: each lane takes Q = 32 / VEC groups
// of VEC (VEC = 8: four groups of eight, the 16-byte path; VEC = 4: eight
// groups of four, slices that share only an 8-byte phase), groups lane +
// 64q of the wave's 64 Q, and issues all Q ND of its loads before the first
// add (indices past the last group clamped to it, so no load waits on a
// lane condition); then the rank-order sum and the division of
// reduce_group per group, the stores of those in range.  With one group of
// eight per lane and batches of one slice, a wave moved 2-6 KiB in 1-3
// dependent round trips: 0.53-0.58 of 8 TB/s.  The unaligned head and the
// tail past the last whole group go one element per lane, as in
// zs_reduce_kernel.
template <class Fmt, int ND, int VEC = 8>
__global__ __launch_bounds__(kWave) void zs_reduce_few_kernel(SliceArgs s, uint64_t n,
                                                              uint32_t head,
                                                              uint16_t *__restrict__ out,
                                                              int32_t *__restrict__ flag) {
    constexpr int Q = 32 / VEC;
    typedef typename HVec<Fmt, VEC>::T hv;
    const float count = (float)ND;
    const uint32_t lane = threadIdx.x;
    const uint64_t gtid = (uint64_t)blockIdx.x * kWave + lane;
    const uint64_t gstride = (uint64_t)gridDim.x * kWave;
    int bad = 0;
    const uint64_t h = head < n ? head : n;
    const uint64_t ngroups = (n - h) / VEC;
    const uint64_t body_end = h + ngroups * VEC;
    if (gtid < h)
        reduce_one<Fmt>(s, ND, gtid, count, out, bad);
    for (uint64_t i = body_end + gtid; i < n; i += gstride)
        reduce_one<Fmt>(s, ND, i, count, out, bad);
    for (uint64_t k0 = (uint64_t)blockIdx.x * kWave * Q; k0 < ngroups; k0 += gstride * Q) {
        hv x[Q][ND];
#pragma unroll
        for (int q = 0; q < Q; q++) {
            const uint64_t g = min(k0 + lane + (uint64_t)kWave * q, ngroups - 1u);
#pragma unroll
            for (int r = 0; r < ND; r++)
                x[q][r] = ld_nt(reinterpret_cast<const hv *>(s.p[r] + h + g * VEC));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < Q; q++) {
            const uint64_t g = k0 + lane + (uint64_t)kWave * q;
            if (g >= ngroups)
                continue;
            hv o;
#pragma unroll
            for (int j = 0; j < VEC; j++) {
                float acc = (float)x[q][0][j];
#pragma unroll
                for (int r = 1; r < ND; r++)
                    acc = acc + (float)x[q][r][j];
                o[j] = (typename Fmt::T)(acc / count);
                const typename Fmt::T oj = o[j];
                uint16_t b;
                memcpy(&b, &oj, 2);
                bad |= bits_nonfinite<Fmt>(b);
            }
            st_through(o, reinterpret_cast<hv *>(out + h + g * VEC));
        }
    }
    raise_flag(flag, bad);
}

// Adds slices r0 .. r0+B-1 (rank order) at a lane's eight single elements
// i0 + 64k into acc; all 8B two-byte loads are issued before the first add.
template <int B, class Fmt>
__device__ __forceinline__ void reduce_batch_single(const SliceArgs &s, uint32_t r0, uint64_t i0,
                                                    bool first, float (&acc)[8]) {
    uint16_t x[B][8];
#pragma unroll
    for (int q = 0; q < B; q++)
#pragma unroll
        for (int k = 0; k < 8; k++)
            x[q][k] = as_global(s.p[r0 + q])[i0 + (uint64_t)kWave * k];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < B; q++)
#pragma unroll
        for (int k = 0; k < 8; k++) {
            typename Fmt::T h;
            memcpy(&h, &x[q][k], 2);
            acc[k] = (first && q == 0) ? (float)h : acc[k] + (float)h;
        }
}

// Slices r0 .. r0+rest-1 (rest = 0-7) at a lane's eight single elements as
// one batch.
template <class Fmt>
__device__ __forceinline__ void reduce_rest_single(const SliceArgs &s, uint32_t r0, uint32_t rest,
                                                   uint64_t i0, float (&acc)[8]) {
    switch (rest) {
#define ZS_REST(R)                                                                                 \
    case R:                                                                                        \
        reduce_batch_single<R, Fmt>(s, r0, i0, r0 == 0, acc);                                     \
        break;
        ZS_REST(1) ZS_REST(2) ZS_REST(3) ZS_REST(4) ZS_REST(5) ZS_REST(6) ZS_REST(7)
#undef ZS_REST
    default:
        break;
    }
}

// The reduction when the slices and the output share no common phase: one
// wave per kTile elements, lane L taking elements L + 64k (k < 8), so every
// two-byte load and store instruction of the wave is one contiguous
// 128-byte range; slices in batches of 8 and then the rest (1-7) in one,
// each batch's loads all in flight before its adds; the sum in rank order and one division, as
// reduce_single.  A partial last tile goes element by element.
template <class Fmt>
__global__ __launch_bounds__(kWave) void zs_reduce_single_kernel(SliceArgs s, uint32_t nd,
                                                                 uint64_t n,
                                                                 uint16_t *__restrict__ out,
                                                                 int32_t *__restrict__ flag) {
    const float count = (float)nd;
    const uint32_t lane = threadIdx.x;
    const uint64_t ntiles = (n + kTile - 1) / kTile;
    int bad = 0;
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t lo = t * kTile;
        if (lo + kTile > n) {
            for (uint64_t i = lo + lane; i < n; i += kWave)
                reduce_one<Fmt>(s, nd, i, count, out, bad);
            continue;
        }
        const uint64_t i0 = lo + lane;
        float acc[8];
        uint32_t r = 0;
        for (; r + 8 <= nd; r += 8)
            reduce_batch_single<8, Fmt>(s, r, i0, r == 0, acc);
        reduce_rest_single<Fmt>(s, r, nd - r, i0, acc);
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const typename Fmt::T o = (typename Fmt::T)(acc[k] / count);
            uint16_t b;
            memcpy(&b, &o, 2);
            bad |= bits_nonfinite<Fmt>(b);
            as_global(out)[i0 + (uint64_t)kWave * k] = b;
        }
    }
    raise_flag(flag, bad);
}

// ---------------------------------------------------------------------------
// Fused stage-2 step over a flat shard: the reduce and the Adam step in one
// pass.  Element i's gradient is exactly what zs_reduce_kernel would store
// (fp32 sum of the slices in rank order, one division by nd, rounded to the
// 16-bit format), widened again and fed to the same Adam element, so results
// are bit-identical to the two kernels run in sequence; the 16-bit gradient
// is stored only if the caller asks for it.  Fmt: fp16 or bfloat16, for the
// slices, the parameter and the gradient alike.
// ---------------------------------------------------------------------------
struct FlatState {
    uint16_t *p;    // 16-bit parameter (written)
    float *w, *m, *v;
    uint16_t *gout; // 16-bit reduced gradient (written), or null
    uint32_t pshift, gshift; // the two outputs' element phase mod 4 at the
                             // vector-aligned elements (the kernels' SHIFT)
};

// One 16-bit output of a full fused tile (lane L: elements 4L..4L+3 of
// each run of 256 from `base`): 8-byte vectors when it is in phase (s 0),
// else shifted.
template <typename V, int Q>
__device__ __forceinline__ void out16_store_tile(uint16_t *dst, uint32_t s, uint64_t base,
                                                 uint32_t lane, const V (&x)[Q]) {
    if (s == 0) {
#pragma unroll
        for (int k = 0; k < Q; k++)
            st_nt(x[k], reinterpret_cast<V *>(dst + base + 4u * kWave * k + 4u * lane));
    } else {
        shifted_store_tile(dst, s, base, lane, x);
    }
}

template <class Fmt>
__device__ __forceinline__ void fused_single(const SliceArgs &s, uint32_t nd, uint64_t i,
                                             float count, const FlatState &F,
                                             const AdamConsts &c, int &bad) {
    const typename Fmt::T gh = (typename Fmt::T)(reduce_single<Fmt>(s, nd, i) / count);
    uint16_t gb;
    memcpy(&gb, &gh, 2);
    bad |= bits_nonfinite<Fmt>(gb);
    if (F.gout != nullptr)
        as_global(F.gout)[i] = gb;
    float w = as_global(F.w)[i], m = as_global(F.m)[i], v = as_global(F.v)[i];
    const typename Fmt::T p = adam_elem<Fmt>((float)gh, w, m, v, c, bad);
    as_global(F.w)[i] = w;
    as_global(F.m)[i] = m;
    as_global(F.v)[i] = v;
    uint16_t pb;
    memcpy(&pb, &p, 2);
    as_global(F.p)[i] = pb;
}

// Adds slices r0 .. r0+B-1 (rank order) at the Q four-element groups
// starting at i[0..Q-1] into acc; all B*Q loads are issued before the first
// add.  With `first`, slice r0 initialises the sums.
template <class Fmt, int B, int Q>
__device__ __forceinline__ void fused_batch(const SliceArgs &s, uint32_t r0, const uint64_t (&i)[Q],
                                            bool first, f32x4 (&acc)[Q]) {
    typedef typename Fmt::V4 hv;
    hv x[B][Q];
#pragma unroll
    for (int q = 0; q < B; q++)
#pragma unroll
        for (int k = 0; k < Q; k++)
            x[q][k] = ld_nt(reinterpret_cast<const hv *>(s.p[r0 + q] + i[k]));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < B; q++)
#pragma unroll
        for (int k = 0; k < Q; k++)
#pragma unroll
            for (int j = 0; j < 4; j++)
                acc[k][j] = (first && q == 0) ? (float)x[0][k][j] : acc[k][j] + (float)x[q][k][j];
}

// Slices r0 .. r0+rest-1 (rest = 1-15) at the Q groups as one batch.
template <class Fmt, int Q>
__device__ __forceinline__ void fused_rest(const SliceArgs &s, uint32_t r0, uint32_t rest,
                                           const uint64_t (&i)[Q], f32x4 (&acc)[Q]) {
    const bool first = r0 == 0;
    switch (rest) {
#define ZS_REST(R)                                                                                 \
    case R:                                                                                        \
        fused_batch<Fmt, R, Q>(s, r0, i, first, acc);                                             \
        break;
        ZS_REST(1) ZS_REST(2) ZS_REST(3) ZS_REST(4) ZS_REST(5) ZS_REST(6) ZS_REST(7) ZS_REST(8)
        ZS_REST(9) ZS_REST(10) ZS_REST(11) ZS_REST(12) ZS_REST(13) ZS_REST(14) ZS_REST(15)
#undef ZS_REST
    default:
        break;
    }
}

// Q four-element groups at i[0..Q-1] (vector-aligned): the fp32 state is
// loaded first, then the slices in batches of 16 and the rest in one; then the
// reduced gradient, the update and the stores.  SHIFT: the 16-bit outputs
// may be out of phase; they are then stored after the state, Q = 2 as a
// full tile from `base`, Q = 1 as groups of the nq lanes from `base`.
template <class Fmt, int Q, bool SHIFT = false>
__device__ __forceinline__ void fused_groups(const SliceArgs &s, uint32_t nd,
                                             const uint64_t (&i)[Q], float count,
                                             const FlatState &F, const AdamConsts &c, int &bad,
                                             uint64_t base = 0, uint32_t nq = 0) {
    f32x4 w[Q], m[Q], v[Q];
#pragma unroll
    for (int k = 0; k < Q; k++) {
        w[k] = ld_nt(reinterpret_cast<const f32x4 *>(F.w + i[k]));
        m[k] = ld_nt(reinterpret_cast<const f32x4 *>(F.m + i[k]));
        v[k] = ld_nt(reinterpret_cast<const f32x4 *>(F.v + i[k]));
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[Q];
    uint32_t r = 0;
    for (; r + 16 <= nd; r += 16)
        fused_batch<Fmt, 16, Q>(s, r, i, r == 0, acc);
    if (r < nd)
        fused_rest<Fmt, Q>(s, r, nd - r, i, acc);
    typename Fmt::V4 gs[Q], ps[Q];
#pragma unroll
    for (int k = 0; k < Q; k++) {
        typename Fmt::V4 g, p;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            g[j] = (typename Fmt::T)(acc[k][j] / count);
            const typename Fmt::T gj = g[j];
            uint16_t gb;
            memcpy(&gb, &gj, 2);
            bad |= bits_nonfinite<Fmt>(gb);
            float ww = w[k][j], mm = m[k][j], vv = v[k][j];
            p[j] = adam_elem<Fmt>((float)gj, ww, mm, vv, c, bad);
            w[k][j] = ww;
            m[k][j] = mm;
            v[k][j] = vv;
        }
        if (!SHIFT && F.gout != nullptr)
            st_nt(g, reinterpret_cast<typename Fmt::V4 *>(F.gout + i[k]));
        st_nt(w[k], reinterpret_cast<f32x4 *>(F.w + i[k]));
        st_nt(m[k], reinterpret_cast<f32x4 *>(F.m + i[k]));
        st_nt(v[k], reinterpret_cast<f32x4 *>(F.v + i[k]));
        if (!SHIFT)
            st_nt(p, reinterpret_cast<typename Fmt::V4 *>(F.p + i[k]));
        gs[k] = g;
        ps[k] = p;
    }
    if constexpr (SHIFT) {
        if constexpr (Q == 1) {
            if (F.pshift == 0)
                st_nt(ps[0], reinterpret_cast<typename Fmt::V4 *>(F.p + i[0]));
            else
                shifted_store_groups(F.p, F.pshift, base, threadIdx.x, nq, ps[0]);
            if (F.gout != nullptr && F.gshift == 0)
                st_nt(gs[0], reinterpret_cast<typename Fmt::V4 *>(F.gout + i[0]));
            else if (F.gout != nullptr)
                shifted_store_groups(F.gout, F.gshift, base, threadIdx.x, nq, gs[0]);
        } else {
            out16_store_tile(F.p, F.pshift, base, threadIdx.x, ps);
            if (F.gout != nullptr)
                out16_store_tile(F.gout, F.gshift, base, threadIdx.x, gs);
        }
    }
}

// The reduction when the slices and the output share an 8-byte phase but
// not a 16-byte one: one wave per kTile elements after the head, each lane
// reducing two groups of four (elements 4L..4L+3 and kTile/2+4L..), so a
// lane keeps as many bytes per slice in flight as on the 16-byte path
// (batches of 16 slices, then the rest in one batch); the
// rank-order sum and the division of reduce_single.  The last, partial tile
// goes by groups of four, then singly; tile 0 also does the head.  With
// xrun != 0 (the grid a multiple of 8 xrun), workgroup b takes, within each
// window of 8 xrun tiles, tile (b mod 8) xrun + (b mod 8 xrun) / 8: the
// workgroups of one XCD (the hardware deals them out in turn, b mod 8) walk
// runs of xrun neighbouring tiles, so the line that two neighbouring tiles
// of a slice off its 128-byte lines share is mostly read once into that
// XCD's L2 instead of once into each of two.
template <class Fmt, bool SHIFT = false>
__global__ __launch_bounds__(kWave) void zs_reduce_vec4_kernel(SliceArgs s, uint32_t nd,
                                                               uint64_t n, uint32_t head,
                                                               uint64_t ntiles,
                                                               uint16_t *__restrict__ out,
                                                               int32_t *__restrict__ flag,
                                                               uint32_t oshift, uint32_t xrun) {
    const float count = (float)nd;
    const uint32_t lane = threadIdx.x;
    const uint64_t h = head < n ? head : n;
    int bad = 0;
    uint64_t b0 = blockIdx.x;
    if (xrun != 0) {
        const uint32_t w = 8u * xrun, within = blockIdx.x % w;
        b0 = (uint64_t)(blockIdx.x / w) * w + (within % 8u) * xrun + within / 8u;
    }
    for (uint64_t b = b0; b < ntiles; b += gridDim.x) {
        if (b == 0 && lane < h)
            reduce_one<Fmt>(s, nd, lane, count, out, bad);
        const uint64_t lo = h + b * kTile;
        if (lo >= n)
            continue;
        const uint64_t hi = min(n, lo + kTile);
        if (hi - lo == kTile) {
            const uint64_t i[2] = {lo + 4u * lane, lo + 4u * lane + kTile / 2};
            f32x4 acc[2];
            uint32_t r = 0;
            for (; r + 16 <= nd; r += 16)
                fused_batch<Fmt, 16, 2>(s, r, i, r == 0, acc);
            if (r < nd)
                fused_rest<Fmt, 2>(s, r, nd - r, i, acc);
            typename Fmt::V4 os[2];
#pragma unroll
            for (int k = 0; k < 2; k++) {
                typename Fmt::V4 o;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    o[j] = (typename Fmt::T)(acc[k][j] / count);
                    const typename Fmt::T oj = o[j];
                    uint16_t ob;
                    memcpy(&ob, &oj, 2);
                    bad |= bits_nonfinite<Fmt>(ob);
                }
                if (!SHIFT)
                    st_through(o, reinterpret_cast<typename Fmt::V4 *>(out + i[k]));
                os[k] = o;
            }
            if (SHIFT)
                shifted_store_tile(out, oshift, lo, lane, os);
            continue;
        }
        const uint32_t nquads = (uint32_t)(hi - lo) / 4u;
        if constexpr (SHIFT) {
            for (uint32_t r0 = 0; r0 < nquads; r0 += kWave) {
                const uint32_t nq = min(nquads - r0, kWave);
                if (lane < nq) {
                    const uint64_t run = lo + 4u * r0;
                    shifted_store_groups(out, oshift, run, lane, nq,
                                         reduce_group_value<Fmt, 4>(s, nd, run + 4u * lane,
                                                                    count, bad));
                }
            }
        } else {
            for (uint32_t q = lane; q < nquads; q += kWave)
                reduce_group<Fmt, 4>(s, nd, lo + 4u * q, count, out, bad);
        }
        const uint64_t t0 = lo + 4u * (uint64_t)nquads;
        if (t0 + lane < hi)
            reduce_one<Fmt>(s, nd, t0 + lane, count, out, bad);
    }
    raise_flag(flag, bad);
}

// Dynamic LDS of the launch: the part of the occupancy reservation that the
// fused kernel uses (1 KiB per one-wave workgroup).
extern __shared__ __attribute__((aligned(16))) unsigned char zs_lds[];

// A full tile with the slices 16-byte aligned: lane L reduces the 8
// consecutive elements 8L..8L+7 (16-byte loads, 1 KiB per wave
// instruction, batches of 16 slices and then the rest in one batch, as
// zs_reduce_kernel), the fp16 gradients go through LDS to
// the Adam tile's mapping (lane L: 4L..4L+3 and kTile/2+4L..), and the
// update runs there.  The fp32 state loads are issued before the slices, or
// with LATE after them (before the LDS exchange).
template <class Fmt, bool LATE, bool SHIFT>
__device__ __forceinline__ void fused_tile8(const SliceArgs &s, uint32_t nd, uint64_t lo,
                                            uint32_t lane, float count, const FlatState &F,
                                            const AdamConsts &c, int &bad) {
    const uint64_t i[2] = {lo + 4u * lane, lo + 4u * lane + kTile / 2};
    f32x4 w[2], m[2], v[2];
    if (!LATE) {
#pragma unroll
        for (int k = 0; k < 2; k++) {
            w[k] = ld_nt(reinterpret_cast<const f32x4 *>(F.w + i[k]));
            m[k] = ld_nt(reinterpret_cast<const f32x4 *>(F.m + i[k]));
            v[k] = ld_nt(reinterpret_cast<const f32x4 *>(F.v + i[k]));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    const uint64_t j = lo + 8u * lane;
    float acc[8];
    uint32_t r = 0;
    for (; r + 16 <= nd; r += 16)
        reduce_batch<8, 16, Fmt>(s, r, j, r == 0, acc);
    if (r < nd)
        reduce_rest<8, Fmt>(s, r, nd - r, j, acc);
    typedef typename Fmt::V8 hv8;
    typedef typename Fmt::V4 hv4;
    hv8 g8;
#pragma unroll
    for (int q = 0; q < 8; q++)
        g8[q] = (typename Fmt::T)(acc[q] / count);
    if (LATE) {
#pragma unroll
        for (int k = 0; k < 2; k++) {
            w[k] = ld_nt(reinterpret_cast<const f32x4 *>(F.w + i[k]));
            m[k] = ld_nt(reinterpret_cast<const f32x4 *>(F.m + i[k]));
            v[k] = ld_nt(reinterpret_cast<const f32x4 *>(F.v + i[k]));
        }
    }
    reinterpret_cast<hv8 *>(zs_lds)[lane] = g8;
    __syncthreads(); // one wave per workgroup: orders the LDS write and reads
    hv4 g[2];
    g[0] = reinterpret_cast<const hv4 *>(zs_lds)[lane];
    g[1] = reinterpret_cast<const hv4 *>(zs_lds)[kWave + lane];
    __syncthreads(); // the next tile of this workgroup rewrites the buffer
    hv4 ps[2];
#pragma unroll
    for (int k = 0; k < 2; k++) {
        hv4 p;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const typename Fmt::T gj = g[k][q];
            uint16_t gb;
            memcpy(&gb, &gj, 2);
            bad |= bits_nonfinite<Fmt>(gb);
            float ww = w[k][q], mm = m[k][q], vv = v[k][q];
            p[q] = adam_elem<Fmt>((float)gj, ww, mm, vv, c, bad);
            w[k][q] = ww;
            m[k][q] = mm;
            v[k][q] = vv;
        }
        if (!SHIFT && F.gout != nullptr)
            st_nt(g[k], reinterpret_cast<hv4 *>(F.gout + i[k]));
        st_nt(w[k], reinterpret_cast<f32x4 *>(F.w + i[k]));
        st_nt(m[k], reinterpret_cast<f32x4 *>(F.m + i[k]));
        st_nt(v[k], reinterpret_cast<f32x4 *>(F.v + i[k]));
        if (!SHIFT)
            st_nt(p, reinterpret_cast<hv4 *>(F.p + i[k]));
        ps[k] = p;
    }
    if constexpr (SHIFT) {
        out16_store_tile(F.p, F.pshift, lo, lane, ps);
        if (F.gout != nullptr)
            out16_store_tile(F.gout, F.gshift, lo, lane, g);
    }
}

// A full tile of the fused step when the slices, parameter and state share
// no common phase: lane L takes elements L + 64k (k < 8), every access
// instruction of the wave contiguous; the fp32 state is loaded first, the
// slices in batches of 8 and then the rest in one (loads in flight before
// the adds), then
// the same per-element reduction, narrowing and update as fused_single.
template <class Fmt>
__device__ __forceinline__ void fused_tile_single(const SliceArgs &s, uint32_t nd, uint64_t lo,
                                                  uint32_t lane, float count,
                                                  const FlatState &F, const AdamConsts &c,
                                                  int &bad) {
    const uint64_t i0 = lo + lane;
    float w[8], m[8], v[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const uint64_t i = i0 + (uint64_t)kWave * k;
        w[k] = as_global(F.w)[i];
        m[k] = as_global(F.m)[i];
        v[k] = as_global(F.v)[i];
    }
    __builtin_amdgcn_sched_barrier(0);
    float acc[8];
    uint32_t r = 0;
    for (; r + 8 <= nd; r += 8)
        reduce_batch_single<8, Fmt>(s, r, i0, r == 0, acc);
    reduce_rest_single<Fmt>(s, r, nd - r, i0, acc);
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const uint64_t i = i0 + (uint64_t)kWave * k;
        const typename Fmt::T gh = (typename Fmt::T)(acc[k] / count);
        uint16_t gb;
        memcpy(&gb, &gh, 2);
        bad |= bits_nonfinite<Fmt>(gb);
        if (F.gout != nullptr)
            as_global(F.gout)[i] = gb;
        const typename Fmt::T p = adam_elem<Fmt>((float)gh, w[k], m[k], v[k], c, bad);
        as_global(F.w)[i] = w[k];
        as_global(F.m)[i] = m[k];
        as_global(F.v)[i] = v[k];
        uint16_t pb;
        memcpy(&pb, &p, 2);
        as_global(F.p)[i] = pb;
    }
}

// One wave per tile of kTile elements after the peeled head (tile 0 also
// does the head).  VEC = 8: full tiles by fused_tile8 (slices 16-byte
// aligned).  VEC = 4: full tiles with each lane reducing its own two groups
// of four (slices 8-byte aligned).  Both: the last partial tile four per
// lane, then singly.  VEC = 1: the tile's elements one at a time.  Tiles
// beyond the grid stride.  LATE: fused_tile8 loads the state after the
// slices.  SHIFT: the parameter or the gradient output is out of the
// others' phase (F.pshift, F.gshift) and is stored shifted.
template <class Fmt, int VEC, bool LATE = false, bool SHIFT = false>
__global__ __launch_bounds__(kWave) void zs_fused_kernel(SliceArgs s, uint32_t nd, uint64_t n,
                                                         uint32_t head, uint64_t ntiles,
                                                         FlatState F, AdamConsts c,
                                                         int32_t *__restrict__ flag) {
    const float count = (float)nd;
    const uint32_t lane = threadIdx.x;
    const uint64_t h = head < n ? head : n;
    int bad = 0;
    for (uint64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        if (b == 0 && lane < h)
            fused_single<Fmt>(s, nd, lane, count, F, c, bad);
        const uint64_t lo = h + b * kTile;
        const uint64_t hi = min(n, lo + kTile);
        if (VEC > 1) {
            if (hi - lo == kTile && VEC == 8) {
                fused_tile8<Fmt, LATE, SHIFT>(s, nd, lo, lane, count, F, c, bad);
            } else if (hi - lo == kTile) {
                const uint64_t i[2] = {lo + 4u * lane, lo + 4u * lane + kTile / 2};
                fused_groups<Fmt, 2, SHIFT>(s, nd, i, count, F, c, bad, lo, kWave);
            } else {
                const uint32_t nquads = (uint32_t)(hi - lo) / 4u;
                if constexpr (SHIFT) {
                    for (uint32_t r0 = 0; r0 < nquads; r0 += kWave) {
                        const uint32_t nq = min(nquads - r0, kWave);
                        if (lane < nq) {
                            const uint64_t run = lo + 4u * r0;
                            const uint64_t i[1] = {run + 4u * lane};
                            fused_groups<Fmt, 1, true>(s, nd, i, count, F, c, bad, run, nq);
                        }
                    }
                } else {
                    for (uint32_t q = lane; q < nquads; q += kWave) {
                        const uint64_t i[1] = {lo + 4u * q};
                        fused_groups<Fmt, 1>(s, nd, i, count, F, c, bad);
                    }
                }
                const uint64_t t0 = lo + 4u * (uint64_t)nquads;
                if (t0 + lane < hi)
                    fused_single<Fmt>(s, nd, t0 + lane, count, F, c, bad);
            }
        } else if (hi - lo == kTile) {
            fused_tile_single<Fmt>(s, nd, lo, lane, count, F, c, bad);
        } else {
            for (uint64_t k = lo + lane; k < hi; k += kWave)
                fused_single<Fmt>(s, nd, k, count, F, c, bad);
        }
    }
    raise_flag(flag, bad);
}

// ---------------------------------------------------------------------------
// Parameter gather: nd shards of S fp16 elements into the full buffer.
// ---------------------------------------------------------------------------
struct GatherArgs {
    const uint16_t *src[ZERO_MAX_SLICES];
    uint8_t vec[ZERO_MAX_SLICES];   // 8, 4, 2 or 1 elements per access; 3: four, the
                                    // source read shifted; 0: in place, skip
    uint8_t head[ZERO_MAX_SLICES];  // leading elements copied singly
    uint8_t shift[ZERO_MAX_SLICES]; // vec 3: the source's element phase mod 4 at
                                    // the destination's vector-aligned elements
};

template <typename V>
__device__ __forceinline__ void copy_vec(const uint16_t *src, uint16_t *dst, uint64_t i) {
    st_nt(ld_nt(reinterpret_cast<const V *>(src + i)), reinterpret_cast<V *>(dst + i));
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Tile j of shard r: after the shard's head (the elements before the
// destination's first 128-byte line), kGatherTile consecutive
// elements.  A full tile has each lane move kGatherTile / (64 VEC) groups
// of VEC elements (lane L's groups at L, L + 64, ...: every wave instruction
// contiguous), all loads before the first store; the shard's last, partial
// tile moves its whole groups of VEC, then single elements.
template <int VEC, typename V>
__device__ __forceinline__ void gather_tile(const uint16_t *src, uint16_t *dst, uint64_t S,
                                            uint32_t head, uint64_t j) {
    const uint32_t lane = threadIdx.x;
    const uint64_t h = head < S ? head : S;
    if (j == 0 && lane < h)
        as_global(dst)[lane] = as_global(src)[lane];
    const uint64_t lo = h + j * zs::kGatherTile;
    if (lo >= S)
        return;
    const uint64_t hi = min(S, lo + zs::kGatherTile);
    if (hi - lo == zs::kGatherTile) {
        constexpr int G = zs::kGatherTile / (kWave * VEC);
        V x[G];
#pragma unroll
        for (int k = 0; k < G; k++)
            x[k] = ld_nt(reinterpret_cast<const V *>(src + lo + (lane + kWave * k) * VEC));
#pragma unroll
        for (int k = 0; k < G; k++)
            st_nt(x[k], reinterpret_cast<V *>(dst + lo + (lane + kWave * k) * VEC));
        return;
    }
    const uint64_t ngroups = (hi - lo) / VEC;
    for (uint64_t q = lane; q < ngroups; q += kWave)
        copy_vec<V>(src, dst, lo + q * VEC);
    for (uint64_t i = lo + ngroups * VEC + lane; i < hi; i += kWave)
        as_global(dst)[i] = as_global(src)[i];
}

// Tile j of shard r when the source is s elements (1-3) out of the
// destination's phase: the tiles of gather_tile's four-element path, each
// lane reading its groups as two whole aligned words of the source
// (load_shifted) and storing them as aligned 8-byte vectors on the
// destination's lines.
__device__ __forceinline__ void gather_tile_shifted(const uint16_t *src, uint16_t *dst,
                                                    uint64_t S, uint32_t head, uint64_t j,
                                                    uint32_t s) {
    const uint32_t lane = threadIdx.x;
    const uint64_t h = head < S ? head : S;
    if (j == 0 && lane < h)
        as_global(dst)[lane] = as_global(src)[lane];
    const uint64_t lo = h + j * zs::kGatherTile;
    if (lo >= S)
        return;
    const uint64_t hi = min(S, lo + zs::kGatherTile);
    if (hi - lo == zs::kGatherTile) {
        constexpr int G = zs::kGatherTile / (kWave * 4);
        uint64_t x[G];
#pragma unroll
        for (int k = 0; k < G; k++)
            x[k] = load_shifted(src, s, lo + (lane + kWave * k) * 4u);
#pragma unroll
        for (int k = 0; k < G; k++)
            st_nt(x[k], reinterpret_cast<uint64_t *>(dst + lo + (lane + kWave * k) * 4u));
        return;
    }
    const uint64_t ngroups = (hi - lo) / 4u;
    for (uint64_t q = lane; q < ngroups; q += kWave)
        st_nt(load_shifted(src, s, lo + q * 4u), reinterpret_cast<uint64_t *>(dst + lo + q * 4u));
    for (uint64_t i = lo + ngroups * 4u + lane; i < hi; i += kWave)
        as_global(dst)[i] = as_global(src)[i];
}

// Grid: x over a shard's tiles (striding when a shard has more than the
// launch's x extent), y over the shards, so consecutive workgroups take
// consecutive tiles of one shard and no workgroup divides to find its
// shard.  Workgroups of a shard that is already in place return at once.
__global__ __launch_bounds__(kWave) void zs_gather_kernel(GatherArgs a, uint64_t S,
                                                          uint64_t tiles_per_shard,
                                                          uint16_t *__restrict__ full) {
    const uint32_t r = blockIdx.y;
    const uint32_t vec = a.vec[r];
    if (vec == 0)
        return; // in place
    const uint16_t *src = a.src[r];
    uint16_t *dst = full + (uint64_t)r * S;
    const uint32_t head = a.head[r];
    for (uint64_t j = blockIdx.x; j < tiles_per_shard; j += gridDim.x) {
        switch (vec) {
        case 8: gather_tile<8, f16x8>(src, dst, S, head, j); break;
        case 4: gather_tile<4, f16x4>(src, dst, S, head, j); break;
        case 3: gather_tile_shifted(src, dst, S, head, j, a.shift[r]); break;
        case 2: gather_tile<2, u16x2>(src, dst, S, head, j); break;
        default: gather_tile<1, uint16_t>(src, dst, S, head, j); break;
        }
    }
}

// ---------------------------------------------------------------------------
// Launch shapes.
// ---------------------------------------------------------------------------

// Dynamic LDS to reserve per one-wave workgroup so that at most `per_cu`
// workgroups fit on a CU: the largest multiple of 256 bytes below
// lds_per_cu / (per_cu + 1/2), so per_cu of them fit with room to spare and
// one more does not.  (On a 160 KiB CU that holds for per_cu up to 27
// except 19 and 21, which admit 20 and 22; the callers ask for neither.)
// Returns 0 (no cap) if the device does not say.
size_t lds_cap_bytes(int device, uint32_t per_cu) {
    int lds_cu = 0, lds_block = 0;
    if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              device) != hipSuccess ||
        hipDeviceGetAttribute(&lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, device) !=
            hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    if (lds_cu <= 0 || per_cu == 0)
        return 0;
    size_t b = (size_t)(2 * (uint64_t)lds_cu / (2 * (uint64_t)per_cu + 1));
    b = b / 256 * 256;
    if (lds_block > 0 && b > (size_t)lds_block)
        b = (size_t)lds_block;
    return b;
}

} // namespace

struct zero_plan {
    zs::TensorDesc *d_tensors;
    zs::Chunk *d_chunks;
    void *d_table;
    zero_plan_stats stats;
    int device;
    size_t lds_cap; // dynamic LDS per Adam workgroup (the occupancy cap)
    bool bf16;      // parameters and gradients are bfloat16 (else fp16)
    bool shifts;    // some tensor has a 16-bit array out of phase
};

namespace {

int plan_create(const zero_tensor *tensors, uint32_t n_tensors, uint32_t chunk_elems, bool bf16,
                zero_plan **out) {
    if (!out)
        return ZERO_EINVAL;
    zs::HostPlan hp;
    int rc = zs::build_host_plan(tensors, n_tensors, chunk_elems, &hp);
    if (rc != ZERO_OK)
        return rc;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return ZERO_EHIP;
    }
    zero_plan *plan = new (std::nothrow) zero_plan;
    if (!plan)
        return ZERO_ENOMEM;
    plan->d_table = nullptr;
    plan->d_tensors = nullptr;
    plan->d_chunks = nullptr;
    plan->stats = hp.stats;
    plan->device = dev;
    plan->lds_cap = lds_cap_bytes(dev, (uint32_t)hp.stats.wg_per_cu);
    plan->bf16 = bf16;
    plan->shifts = zs::any_shift(hp.tensors.data(), hp.tensors.size());
    const size_t tb = hp.tensors.size() * sizeof(zs::TensorDesc);
    const size_t cb = hp.chunks.size() * sizeof(zs::Chunk);
    if (tb + cb > 0) {
        if (hipMalloc(&plan->d_table, tb + cb) != hipSuccess) {
            (void)hipGetLastError();
            delete plan;
            return ZERO_ENOMEM;
        }
        plan->d_tensors = (zs::TensorDesc *)plan->d_table;
        plan->d_chunks = (zs::Chunk *)((char *)plan->d_table + tb);
        if (hipMemcpy(plan->d_tensors, hp.tensors.data(), tb, hipMemcpyHostToDevice) != hipSuccess ||
            hipMemcpy(plan->d_chunks, hp.chunks.data(), cb, hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipGetLastError();
            (void)hipFree(plan->d_table);
            delete plan;
            return ZERO_EHIP;
        }
    }
    *out = plan;
    return ZERO_OK;
}

} // namespace

extern "C" int zero_plan_create(const zero_tensor *tensors, uint32_t n_tensors,
                                uint32_t chunk_elems, zero_plan **out) {
    return plan_create(tensors, n_tensors, chunk_elems, false, out);
}

extern "C" int zero_plan_create_bf16(const zero_tensor *tensors, uint32_t n_tensors,
                                     uint32_t chunk_elems, zero_plan **out) {
    return plan_create(tensors, n_tensors, chunk_elems, true, out);
}

extern "C" int zero_plan_stats_of(const zero_plan *plan, zero_plan_stats *out) {
    if (!plan || !out)
        return ZERO_EINVAL;
    *out = plan->stats;
    return ZERO_OK;
}

extern "C" int zero_plan_destroy(zero_plan *plan) {
    if (!plan)
        return ZERO_OK;
    int rc = ZERO_OK;
    if (plan->d_table && hipFree(plan->d_table) != hipSuccess) {
        (void)hipGetLastError();
        rc = ZERO_EHIP;
    }
    delete plan;
    return rc;
}

namespace {

// The Adam launch over a device table (descriptors and chunks) with the
// given statistics: one one-wave workgroup per Adam tile, dispatched in
// order and balanced over the CUs by the hardware; only tables beyond
// kMaxGrid tiles stride.
template <class Fmt, uint32_t TILE>
void launch_adam_kernel(bool shifts, uint32_t grid, size_t lds, hipStream_t st,
                        const TensorDesc *d_tensors, const Chunk *d_chunks, uint64_t n_virtual,
                        uint32_t tpc, const AdamConsts &c, int32_t *flag, const int32_t *skip,
                        const int32_t *log2_scale) {
    if (shifts)
        hipLaunchKernelGGL((zs_adam_kernel<Fmt, TILE, true>), dim3(grid), dim3(kWave), lds, st,
                           d_tensors, d_chunks, n_virtual, tpc, c, flag, skip, log2_scale);
    else
        hipLaunchKernelGGL((zs_adam_kernel<Fmt, TILE, false>), dim3(grid), dim3(kWave), lds, st,
                           d_tensors, d_chunks, n_virtual, tpc, c, flag, skip, log2_scale);
}

// shifts: some tensor of the table has a 16-bit array out of phase (the
// kernel variant with the shifted modes; without, the in-phase tile code
// is compiled alone).
int launch_adam_table(const TensorDesc *d_tensors, const Chunk *d_chunks,
                      const zero_plan_stats &stats, size_t lds, bool bf16, bool shifts,
                      const AdamConsts &c, int32_t *flag, const int32_t *skip,
                      const int32_t *log2_scale, hipStream_t st) {
    const uint32_t tile = (uint32_t)stats.tile_elems;
    const uint32_t tpc = (uint32_t)(stats.chunk_elems / tile);
    const uint64_t n_virtual = stats.n_chunks * tpc;
    const uint32_t grid = (uint32_t)(n_virtual < zs::kMaxGrid ? n_virtual : zs::kMaxGrid);
    if (bf16 && tile == kAdamTileFine)
        launch_adam_kernel<FmtBF16, kAdamTileFine>(shifts, grid, lds, st, d_tensors, d_chunks,
                                                   n_virtual, tpc, c, flag, skip, log2_scale);
    else if (bf16)
        launch_adam_kernel<FmtBF16, kTile>(shifts, grid, lds, st, d_tensors, d_chunks, n_virtual,
                                           tpc, c, flag, skip, log2_scale);
    else if (tile == kAdamTileFine)
        launch_adam_kernel<FmtF16, kAdamTileFine>(shifts, grid, lds, st, d_tensors, d_chunks,
                                                  n_virtual, tpc, c, flag, skip, log2_scale);
    else
        launch_adam_kernel<FmtF16, kTile>(shifts, grid, lds, st, d_tensors, d_chunks, n_virtual,
                                          tpc, c, flag, skip, log2_scale);
    if (hipGetLastError() != hipSuccess)
        return ZERO_EHIP;
    return ZERO_OK;
}

// The fp32 constants of step t, checked as zero_adam_scalars checks them.
int adam_consts(const zero_adam_hparams *hp, uint64_t t, AdamConsts *c) {
    float s[8];
    const int rc = zero_adam_scalars(hp, t, s);
    if (rc != ZERO_OK)
        return rc;
    *c = {s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7], 1.0f};
    return ZERO_OK;
}

int current_device(int *dev) {
    if (hipGetDevice(dev) != hipSuccess) {
        (void)hipGetLastError();
        return ZERO_EHIP;
    }
    return ZERO_OK;
}

} // namespace

static int adam_step_launch(const zero_plan *plan, const zero_adam_hparams *hp, uint64_t t,
                            int32_t *nonfinite_flag, const int32_t *skip_if_nonzero,
                            const int32_t *log2_scale, void *stream) {
    if (!plan || !hp)
        return ZERO_EINVAL;
    if (nonfinite_flag != nullptr && (const void *)nonfinite_flag == (const void *)skip_if_nonzero)
        return ZERO_EINVAL;
    AdamConsts c;
    int rc = adam_consts(hp, t, &c);
    if (rc != ZERO_OK)
        return rc;
    if (plan->stats.n_chunks == 0)
        return ZERO_OK;
    int dev = -1;
    if ((rc = current_device(&dev)) != ZERO_OK)
        return rc;
    if (dev != plan->device)
        return ZERO_EINVAL;
    return launch_adam_table(plan->d_tensors, plan->d_chunks, plan->stats, plan->lds_cap,
                             plan->bf16, plan->shifts, c, nonfinite_flag, skip_if_nonzero,
                             log2_scale, (hipStream_t)stream);
}

extern "C" int zero_adam_step(const zero_plan *plan, const zero_adam_hparams *hp, uint64_t t,
                              int32_t *nonfinite_flag, const int32_t *skip_if_nonzero,
                              void *stream) {
    return adam_step_launch(plan, hp, t, nonfinite_flag, skip_if_nonzero, nullptr, stream);
}

// true when the 4-byte word at p lies inside the loss-scale record at s
static bool inside_scale(const void *p, const zero_loss_scale *s) {
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)s;
    return p != nullptr && a + 4 > b && a < b + sizeof(zero_loss_scale);
}

extern "C" int zero_adam_step_scaled(const zero_plan *plan, const zero_adam_hparams *hp,
                                     uint64_t t, const zero_loss_scale *scale,
                                     int32_t *nonfinite_flag, const int32_t *skip_if_nonzero,
                                     void *stream) {
    if (!scale || (uintptr_t)scale % 4 || inside_scale(nonfinite_flag, scale) ||
        inside_scale(skip_if_nonzero, scale))
        return ZERO_EINVAL;
    return adam_step_launch(plan, hp, t, nonfinite_flag, skip_if_nonzero, &scale->log2_scale,
                            stream);
}

// One update of the dynamic loss scale from the step's non-finite flag, by
// one thread; the flag is then cleared for the next step.
__global__ __launch_bounds__(kWave) void zs_loss_scale_kernel(zero_loss_scale *__restrict__ s,
                                                              int32_t *__restrict__ flag,
                                                              uint32_t interval, int32_t lo,
                                                              int32_t hi) {
    if (threadIdx.x != 0)
        return;
    zero_loss_scale st = *s;
    if (*flag != 0) {
        st.log2_scale = (int32_t)max((int64_t)lo, (int64_t)st.log2_scale - 1);
        st.good_steps = 0;
        st.skipped_steps += 1;
    } else {
        st.applied_steps += 1;
        st.good_steps += 1;
        if (st.good_steps >= interval) {
            st.log2_scale = (int32_t)min((int64_t)hi, (int64_t)st.log2_scale + 1);
            st.good_steps = 0;
        }
    }
    *s = st;
    *flag = 0;
}

extern "C" int zero_loss_scale_update(zero_loss_scale *scale, int32_t *nonfinite_flag,
                                      uint32_t interval, int32_t min_log2, int32_t max_log2,
                                      void *stream) {
    if (!scale || !nonfinite_flag || (uintptr_t)scale % 4 || (uintptr_t)nonfinite_flag % 4 ||
        inside_scale(nonfinite_flag, scale) || interval == 0 || min_log2 > max_log2 ||
        min_log2 < -ZERO_LOG2_SCALE_MAX || max_log2 > ZERO_LOG2_SCALE_MAX)
        return ZERO_EINVAL;
    hipLaunchKernelGGL(zs_loss_scale_kernel, dim3(1), dim3(kWave), 0, (hipStream_t)stream, scale,
                       nonfinite_flag, interval, min_log2, max_log2);
    if (hipGetLastError() != hipSuccess)
        return ZERO_EHIP;
    return ZERO_OK;
}

namespace {

template <class Fmt>
int reduce_grad_shard(const void *const *slices_f16, uint32_t nd, uint64_t n, void *out_f16,
                      int32_t *nonfinite_flag, void *stream) {
    if (!slices_f16 || !out_f16 || nd == 0 || nd > ZERO_MAX_SLICES)
        return ZERO_EINVAL;
    uint64_t bytes;
    if (__builtin_mul_overflow(n, (uint64_t)2, &bytes))
        return ZERO_EOVERFLOW;
    const uintptr_t o = (uintptr_t)out_f16;
    if (o % 2 || o + bytes < o)
        return ZERO_EINVAL;
    SliceArgs args;
    uintptr_t addr[ZERO_MAX_SLICES + 1];
    for (uint32_t r = 0; r < nd; r++) {
        const uintptr_t a = (uintptr_t)slices_f16[r];
        if (!a || a % 2 || a + bytes < a)
            return ZERO_EINVAL;
        // the output must not overlap any slice
        if (n > 0 && a < o + bytes && o < a + bytes)
            return ZERO_EINVAL;
        args.p[r] = (const uint16_t *)slices_f16[r];
        addr[r] = a;
    }
    for (uint32_t r = nd; r < ZERO_MAX_SLICES; r++)
        args.p[r] = nullptr;
    if (n == 0)
        return ZERO_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return ZERO_EHIP;
    }
    addr[nd] = o;
    uint32_t vec, head;
    zs::pick_vector_path(addr, (int)nd + 1, nullptr, 0, 8, &vec, &head);
    // the output alone out of the slices' phase (a parameter view at an
    // offset that is not a multiple of four elements, which the fused
    // route reduces into): the slices' path, the output stored shifted,
    // on outputs of kTileAlignMinElems or more, as the Adam step does
    uint32_t oshift = 0;
    if (vec == 1 && n >= zs::kTileAlignMinElems) {
        uint32_t vs, hs;
        zs::pick_vector_path(addr, (int)nd, nullptr, 0, 8, &vs, &hs);
        const uint32_t sh = (uint32_t)((o / 2u + hs) % 4u);
        if (vs > 1 && sh != 0) {
            vec = vs;
            head = hs;
            oshift = sh;
        }
    }
    // 16-byte path: one vector group per lane, one wave per workgroup;
    // 8-byte path: one 512-element tile per wave (two groups per lane);
    // single elements: one 512-element tile per wave, half the bytes per
    // wave in flight, so more workgroups stay resident (reduce_per_cu_path)
    const uint64_t hh = head < n ? head : n;
    const uint64_t tiles4 = (n - hh + kTile - 1) / kTile + (n == hh ? 1 : 0);
    const uint64_t want = vec == 8 ? ((n - hh) / 8 + 1 + kWave - 1) / kWave
                          : vec == 4 ? tiles4 : (n + kTile - 1) / kTile;
    uint32_t grid = (uint32_t)(want < zs::kMaxGrid ? want : zs::kMaxGrid);
    const uint32_t per_cu = zs::reduce_per_cu_path(nd, vec);
    // the 8-byte path's tiles in runs per XCD: a grid of whole windows
    const uint32_t xrun = vec == 4 ? zs::reduce_vec4_run(nd) : 0u;
    if (xrun != 0)
        grid = (grid + 8u * xrun - 1u) / (8u * xrun) * (8u * xrun);
    const size_t lds = lds_cap_bytes(dev, per_cu);
    hipStream_t st = (hipStream_t)stream;
    uint16_t *out = (uint16_t *)out_f16;
    if ((vec == 8 || vec == 4) && oshift == 0 && nd <= 3) {
        // 1-3 slices: 32 elements per lane, all loads in flight at once
        const uint64_t groups = (n - hh) / vec;
        const uint64_t per_wave = (uint64_t)(32u / vec) * kWave;
        const uint64_t w4 = (groups + per_wave - 1) / per_wave;
        const uint64_t wf = w4 > 0 ? w4 : 1;
        const uint32_t gf = (uint32_t)(wf < zs::kMaxGrid ? wf : zs::kMaxGrid);
        const size_t lf = lds_cap_bytes(dev, zs::reduce_per_cu_few(nd, vec));
#define ZS_FEW(ND, V)                                                                              \
    hipLaunchKernelGGL((zs_reduce_few_kernel<Fmt, ND, V>), dim3(gf), dim3(kWave), lf, st, args, n, \
                       head, out, nonfinite_flag)
        if (vec == 8) {
            if (nd == 1)
                ZS_FEW(1, 8);
            else if (nd == 2)
                ZS_FEW(2, 8);
            else
                ZS_FEW(3, 8);
        } else {
            if (nd == 1)
                ZS_FEW(1, 4);
            else if (nd == 2)
                ZS_FEW(2, 4);
            else
                ZS_FEW(3, 4);
        }
#undef ZS_FEW
        if (hipGetLastError() != hipSuccess)
            return ZERO_EHIP;
        return ZERO_OK;
    }
    if (vec == 8 && oshift != 0)
        hipLaunchKernelGGL((zs_reduce_kernel<Fmt, 8, true>), dim3(grid), dim3(kWave), lds, st,
                           args, nd, n, head, out, nonfinite_flag, oshift);
    else if (vec == 8)
        hipLaunchKernelGGL((zs_reduce_kernel<Fmt, 8>), dim3(grid), dim3(kWave), lds, st, args, nd,
                           n, head, out, nonfinite_flag, 0u);
    else if (vec == 4 && oshift != 0)
        hipLaunchKernelGGL((zs_reduce_vec4_kernel<Fmt, true>), dim3(grid), dim3(kWave), lds, st,
                           args, nd, n, head, tiles4, out, nonfinite_flag, oshift, xrun);
    else if (vec == 4)
        hipLaunchKernelGGL((zs_reduce_vec4_kernel<Fmt>), dim3(grid), dim3(kWave), lds, st, args,
                           nd, n, head, tiles4, out, nonfinite_flag, 0u, xrun);
    else
        hipLaunchKernelGGL((zs_reduce_single_kernel<Fmt>), dim3(grid), dim3(kWave), lds, st, args,
                           nd, n, out, nonfinite_flag);
    if (hipGetLastError() != hipSuccess)
        return ZERO_EHIP;
    return ZERO_OK;
}

} // namespace

extern "C" int zero_reduce_grad_shard(const void *const *slices_f16, uint32_t nd, uint64_t n,
                                      void *out_f16, int32_t *nonfinite_flag, void *stream) {
    return reduce_grad_shard<FmtF16>(slices_f16, nd, n, out_f16, nonfinite_flag, stream);
}

extern "C" int zero_reduce_grad_shard_bf16(const void *const *slices_bf16, uint32_t nd,
                                           uint64_t n, void *out_bf16, int32_t *nonfinite_flag,
                                           void *stream) {
    return reduce_grad_shard<FmtBF16>(slices_bf16, nd, n, out_bf16, nonfinite_flag, stream);
}

namespace {

// The Adam step over one flat tensor (p, g, w, m, v of n elements) with
// zs_adam_flat_kernel: the plan builder's access path and tile rule for a
// one-tensor plan (256-element tiles on the vector path, else 512), and
// its occupancy cap.
template <class Fmt>
int adam_flat_launch(uint16_t *p, const uint16_t *g, float *w, float *m, float *v, uint64_t n,
                     const AdamConsts &c, int dev, hipStream_t st) {
    TensorDesc T;
    memset(&T, 0, sizeof(T));
    T.p = p;
    T.g = g;
    T.w = w;
    T.m = m;
    T.v = v;
    T.n = n;
    const uintptr_t a32[3] = {(uintptr_t)w, (uintptr_t)m, (uintptr_t)v};
    zs::adam_access_path((uintptr_t)p, (uintptr_t)g, a32, n, &T);
    const uint32_t tile = T.vec == 4 ? kAdamTileFine : kTile;
    // tiles: the first holds the peeled head (vector path) and up to `tile`
    // elements, every later one `tile` elements, the last what is left
    const uint64_t h = T.vec == 4 && T.head < n ? T.head : 0;
    const uint64_t ntiles = n == h ? 1 : (n - h + tile - 1) / tile;
    const uint64_t first = n < h + tile ? n : h + tile;
    const uint64_t last = ntiles == 1 ? first : n - h - (ntiles - 1) * tile;
    const uint32_t grid = (uint32_t)(ntiles < zs::kMaxGrid ? ntiles : zs::kMaxGrid);
    const size_t lds = lds_cap_bytes(dev, zs::adam_per_cu(tile));
    const bool shifts = zs::any_shift(&T, 1);
    if (tile == kAdamTileFine && shifts)
        hipLaunchKernelGGL((zs_adam_flat_kernel<Fmt, kAdamTileFine, true>), dim3(grid),
                           dim3(kWave), lds, st, T, ntiles, (uint32_t)first, (uint32_t)last, c,
                           nullptr);
    else if (tile == kAdamTileFine)
        hipLaunchKernelGGL((zs_adam_flat_kernel<Fmt, kAdamTileFine, false>), dim3(grid),
                           dim3(kWave), lds, st, T, ntiles, (uint32_t)first, (uint32_t)last, c,
                           nullptr);
    else if (shifts)
        hipLaunchKernelGGL((zs_adam_flat_kernel<Fmt, kTile, true>), dim3(grid), dim3(kWave), lds,
                           st, T, ntiles, (uint32_t)first, (uint32_t)last, c, nullptr);
    else
        hipLaunchKernelGGL((zs_adam_flat_kernel<Fmt, kTile, false>), dim3(grid), dim3(kWave), lds,
                           st, T, ntiles, (uint32_t)first, (uint32_t)last, c, nullptr);
    if (hipGetLastError() != hipSuccess)
        return ZERO_EHIP;
    return ZERO_OK;
}

template <class Fmt>
int reduce_adam_step(const void *const *slices_f16, uint32_t nd, uint64_t n, void *param_f16,
                     float *master, float *m, float *v, void *grad_out_f16,
                     const zero_adam_hparams *hp, uint64_t t, int32_t *nonfinite_flag,
                     void *stream) {
    if (!slices_f16 || nd == 0 || nd > ZERO_MAX_SLICES || !hp)
        return ZERO_EINVAL;
    float sc[8];
    int rc = zero_adam_scalars(hp, t, sc);
    if (rc != ZERO_OK)
        return rc;
    uint64_t b2, b4;
    if (__builtin_mul_overflow(n, (uint64_t)2, &b2) || __builtin_mul_overflow(n, (uint64_t)4, &b4))
        return ZERO_EOVERFLOW;
    if (n == 0)
        return ZERO_OK;
    const uintptr_t p = (uintptr_t)param_f16, go = (uintptr_t)grad_out_f16;
    const uintptr_t w = (uintptr_t)master, mm = (uintptr_t)m, vv = (uintptr_t)v;
    if (!p || !w || !mm || !vv || p % 2 || go % 2 || (w | mm | vv) % 4)
        return ZERO_EINVAL;
    std::vector<zs::Range> ranges;
    ranges.reserve(nd + 5);
    SliceArgs args;
    uintptr_t a16[ZERO_MAX_SLICES + 2];
    for (uint32_t r = 0; r < nd; r++) {
        const uintptr_t a = (uintptr_t)slices_f16[r];
        if (!a || a % 2)
            return ZERO_EINVAL;
        args.p[r] = (const uint16_t *)slices_f16[r];
        a16[r] = a;
        ranges.push_back({a, a + b2, false});
    }
    for (uint32_t r = nd; r < ZERO_MAX_SLICES; r++)
        args.p[r] = nullptr;
    int n16 = (int)nd;
    a16[n16++] = p;
    ranges.push_back({p, p + b2, true});
    if (go) {
        a16[n16++] = go;
        ranges.push_back({go, go + b2, true});
    }
    for (uintptr_t a : {w, mm, vv})
        ranges.push_back({a, a + b4, true});
    for (const zs::Range &x : ranges)
        if (x.hi < x.lo)
            return ZERO_EOVERFLOW;
    if (zs::writes_overlap(ranges))
        return ZERO_EINVAL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return ZERO_EHIP;
    }
    const AdamConsts c = {sc[0], sc[1], sc[2], sc[3], sc[4], sc[5], sc[6], sc[7], 1.0f};
    if (nd >= zs::kFusedSplitSlices) {
        // The reduce into the gradient output, or without one into the
        // parameter array (every element of which the Adam step then reads
        // as its gradient before writing the new parameter in its place),
        // then the Adam step over it: the same values as the fused kernel.
        void *gdst = grad_out_f16 != nullptr ? grad_out_f16 : param_f16;
        rc = reduce_grad_shard<Fmt>(slices_f16, nd, n, gdst, nonfinite_flag, stream);
        if (rc != ZERO_OK)
            return rc;
        return adam_flat_launch<Fmt>((uint16_t *)param_f16, (const uint16_t *)gdst, master, m, v,
                                     n, c, dev, (hipStream_t)stream);
    }
    // Access path: a common phase h (elements peeled singly) after which the
    // slices are 16-byte aligned (VEC 8) or 8-byte aligned (VEC 4), the fp16
    // outputs 8-byte and the fp32 state 16-byte aligned; else single elements.
    uint32_t vec = 1, head = 0;
    for (uint32_t want : {8u, 4u}) {
        for (uint32_t h = 0; h < want && vec == 1; h++) {
            bool ok = (w + 4u * h) % 16 == 0 && (mm + 4u * h) % 16 == 0 &&
                      (vv + 4u * h) % 16 == 0;
            for (uint32_t r = 0; r < nd && ok; r++)
                ok = (a16[r] + 2u * h) % (2u * want) == 0;
            for (int k = (int)nd; k < n16 && ok; k++)
                ok = (a16[k] + 2u * h) % 8 == 0;
            if (ok) {
                vec = want;
                head = h;
            }
        }
        if (vec != 1)
            break;
    }
    // Only the outputs out of phase (a parameter view at an offset that is
    // not a multiple of four elements): the same paths with the outputs'
    // stores shifted, on shards of kTileAlignMinElems or more, as the Adam
    // plan does.
    bool shift = false;
    uint32_t pshift = 0, gshift = 0;
    if (vec == 1 && n >= zs::kTileAlignMinElems) {
        for (uint32_t want : {8u, 4u}) {
            for (uint32_t h = 0; h < want && vec == 1; h++) {
                bool ok = (w + 4u * h) % 16 == 0 && (mm + 4u * h) % 16 == 0 &&
                          (vv + 4u * h) % 16 == 0;
                for (uint32_t r = 0; r < nd && ok; r++)
                    ok = (a16[r] + 2u * h) % (2u * want) == 0;
                if (ok) {
                    vec = want;
                    head = h;
                }
            }
            if (vec != 1)
                break;
        }
        if (vec != 1) {
            shift = true;
            pshift = (uint32_t)((p / 2u + head) % 4u);
            gshift = go ? (uint32_t)((go / 2u + head) % 4u) : 0u;
        }
    }
    const uint64_t h = head < n ? head : n;
    const uint64_t ntiles = (n - h + kTile - 1) / kTile + (n == h ? 1 : 0);
    const uint32_t grid = (uint32_t)(ntiles < zs::kMaxGrid ? ntiles : zs::kMaxGrid);
    // the 16-byte path loads the state after the slices when fewer than 16
    // are in flight per batch
    const bool late = vec == 8 && zs::fused_state_late(nd);
    size_t lds = lds_cap_bytes(dev, zs::fused_per_cu(nd, late, vec));
    if (lds < 2u * kTile)
        lds = 2u * kTile; // the fp16 exchange buffer of fused_tile8
    const FlatState F = {(uint16_t *)param_f16, master, m, v, (uint16_t *)grad_out_f16, pshift,
                         gshift};
    hipStream_t st = (hipStream_t)stream;
    if (vec == 8 && late && shift)
        hipLaunchKernelGGL((zs_fused_kernel<Fmt, 8, true, true>), dim3(grid), dim3(kWave), lds,
                           st, args, nd, n, head, ntiles, F, c, nonfinite_flag);
    else if (vec == 8 && late)
        hipLaunchKernelGGL((zs_fused_kernel<Fmt, 8, true>), dim3(grid), dim3(kWave), lds, st, args,
                           nd, n, head, ntiles, F, c, nonfinite_flag);
    else if (vec == 8 && shift)
        hipLaunchKernelGGL((zs_fused_kernel<Fmt, 8, false, true>), dim3(grid), dim3(kWave), lds,
                           st, args, nd, n, head, ntiles, F, c, nonfinite_flag);
    else if (vec == 8)
        hipLaunchKernelGGL((zs_fused_kernel<Fmt, 8>), dim3(grid), dim3(kWave), lds, st, args, nd,
                           n, head, ntiles, F, c, nonfinite_flag);
    else if (vec == 4 && shift)
        hipLaunchKernelGGL((zs_fused_kernel<Fmt, 4, false, true>), dim3(grid), dim3(kWave), lds,
                           st, args, nd, n, head, ntiles, F, c, nonfinite_flag);
    else if (vec == 4)
        hipLaunchKernelGGL((zs_fused_kernel<Fmt, 4>), dim3(grid), dim3(kWave), lds, st, args, nd,
                           n, head, ntiles, F, c, nonfinite_flag);
    else
        hipLaunchKernelGGL((zs_fused_kernel<Fmt, 1>), dim3(grid), dim3(kWave), lds, st, args, nd,
                           n, 0u, ntiles, F, c, nonfinite_flag);
    if (hipGetLastError() != hipSuccess)
        return ZERO_EHIP;
    return ZERO_OK;
}

} // namespace

extern "C" int zero_reduce_adam_step(const void *const *slices_f16, uint32_t nd, uint64_t n,
                                     void *param_f16, float *master, float *m, float *v,
                                     void *grad_out_f16, const zero_adam_hparams *hp,
                                     uint64_t t, int32_t *nonfinite_flag, void *stream) {
    return reduce_adam_step<FmtF16>(slices_f16, nd, n, param_f16, master, m, v, grad_out_f16,
                                    hp, t, nonfinite_flag, stream);
}

extern "C" int zero_reduce_adam_step_bf16(const void *const *slices_bf16, uint32_t nd,
                                          uint64_t n, void *param_bf16, float *master, float *m,
                                          float *v, void *grad_out_bf16,
                                          const zero_adam_hparams *hp, uint64_t t,
                                          int32_t *nonfinite_flag, void *stream) {
    return reduce_adam_step<FmtBF16>(slices_bf16, nd, n, param_bf16, master, m, v,
                                     grad_out_bf16, hp, t, nonfinite_flag, stream);
}

extern "C" int zero_gather_shards(const void *const *shards_f16, uint32_t nd, uint64_t shard_len,
                                  void *full_f16, void *stream) {
    if (!shards_f16 || !full_f16 || nd == 0 || nd > ZERO_MAX_SLICES)
        return ZERO_EINVAL;
    uint64_t sb, fb;
    if (__builtin_mul_overflow(shard_len, (uint64_t)2, &sb) ||
        __builtin_mul_overflow(sb, (uint64_t)nd, &fb))
        return ZERO_EOVERFLOW;
    const uintptr_t f = (uintptr_t)full_f16;
    if (f % 2 || f + fb < f)
        return ZERO_EINVAL;
    GatherArgs args;
    uint32_t moving = 0;
    for (uint32_t r = 0; r < nd; r++) {
        const uintptr_t s = (uintptr_t)shards_f16[r];
        if (!s || s % 2 || s + sb < s)
            return ZERO_EINVAL;
        const uintptr_t d = f + (uintptr_t)r * sb;
        args.src[r] = (const uint16_t *)shards_f16[r];
        args.head[r] = 0;
        args.shift[r] = 0;
        if (s == d) {
            args.vec[r] = 0; // already in place
            continue;
        }
        // a shard that moves must not overlap the buffer it is copied into
        if (shard_len > 0 && s < f + fb && f < s + sb)
            return ZERO_EINVAL;
        // widest access for which source and destination share a phase; the
        // head (fewer than 64 elements, copied singly) puts the destination
        // of every tile on a 128-byte line, so no two workgroups write parts
        // of one line (the source keeps its phase relative to it)
        uint32_t vec = 1;
        for (uint32_t w : {8u, 4u, 2u}) {
            if ((s - d) % (2u * w) == 0) {
                vec = w;
                break;
            }
        }
        const uint32_t head = (uint32_t)(((zs::kLine - d % zs::kLine) % zs::kLine) / 2u);
        if (vec < 4 && shard_len >= zs::kTileAlignMinElems) {
            // out of 4-element phase: four at a time, the source read shifted
            vec = 3;
            args.shift[r] = (uint8_t)((s / 2u + head) % 4u);
        }
        args.vec[r] = (uint8_t)vec;
        args.head[r] = (uint8_t)head;
        moving++;
    }
    for (uint32_t r = nd; r < ZERO_MAX_SLICES; r++) {
        args.src[r] = nullptr;
        args.vec[r] = 0;
        args.head[r] = 0;
        args.shift[r] = 0;
    }
    if (shard_len == 0 || moving == 0)
        return ZERO_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return ZERO_EHIP;
    }
    // tiles per shard, with room for a head of up to 63 elements; one
    // workgroup per tile and shard, kGatherPerCU of them resident per CU
    const uint64_t tps = (shard_len + zs::kLine / 2 - 1 + zs::kGatherTile - 1) / zs::kGatherTile;
    const uint32_t gx = (uint32_t)(tps < zs::kMaxGrid ? tps : zs::kMaxGrid);
    const size_t lds = lds_cap_bytes(dev, zs::kGatherPerCU);
    hipLaunchKernelGGL(zs_gather_kernel, dim3(gx, nd), dim3(kWave), lds, (hipStream_t)stream,
                       args, shard_len, tps, (uint16_t *)full_f16);
    if (hipGetLastError() != hipSuccess)
        return ZERO_EHIP;
    return ZERO_OK;
}

// ---------------------------------------------------------------------------
// The Adam step without a plan and without allocation: the chunk table is
// rebuilt on the device at every call in a fixed array, then the Adam kernel
// above runs over it.
// ---------------------------------------------------------------------------

// The table of zero_adam_step_noalloc: descriptors, then chunks.  One copy
// per device, held until the process ends.  In host code this name is a
// stand-in, not a device address: the host only ever uses the address that
// hipGetSymbolAddress returns for the current device (noalloc_table below).
static __device__ __align__(256) unsigned char scratch[ZERO_NOALLOC_SCRATCH_BYTES];

namespace {

// Tensors whose descriptors one staging launch carries in its arguments
// (2 KiB of descriptors and 264 bytes of chunk indices).
constexpr uint32_t kStageBatch = 32;

struct StageArgs {
    TensorDesc d[kStageBatch];
    uint64_t chunk0[kStageBatch + 1]; // table index of each tensor's first
                                      // chunk; chunk0[count]: one past the last
};

// Writes the descriptors of tensors first .. first + count - 1 at their
// places in the table and every chunk record of theirs, with the plan
// builder's chunk formulas (zs::chunk_of).  Plain vector stores.
__global__ __launch_bounds__(256) void zs_stage_table_kernel(StageArgs a, uint32_t first,
                                                             uint32_t count, uint64_t C,
                                                             TensorDesc *__restrict__ tensors,
                                                             Chunk *__restrict__ chunks) {
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    if (tid < count)
        tensors[first + tid] = a.d[tid];
    const uint64_t hi = a.chunk0[count];
    for (uint64_t c = a.chunk0[0] + tid; c < hi; c += stride) {
        uint32_t k = 0;
        while (k + 1 < count && a.chunk0[k + 1] <= c)
            k++;
        chunks[c] = zs::chunk_of(a.d[k], first + k, C, c - a.chunk0[k]);
    }
}

// Device address of the table array on device `dev`, taken once per device
// with that device current.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_table_addr[kMaxDevices];
std::mutex g_table_mu;

int noalloc_table(int dev, unsigned char **out) {
    if (dev < 0 || dev >= kMaxDevices)
        return ZERO_EHIP;
    void *p = g_table_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_table_mu);
        p = g_table_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
                (void)hipGetLastError();
                return ZERO_EHIP;
            }
            g_table_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = (unsigned char *)p;
    return ZERO_OK;
}

} // namespace

extern "C" int zero_adam_step_noalloc(const zero_tensor *tensors, uint32_t n_tensors,
                                      const zero_adam_hparams *hp, uint64_t t,
                                      int32_t *nonfinite_flag, const int32_t *skip_if_nonzero,
                                      void *stream) {
    if (!hp || (n_tensors > 0 && !tensors))
        return ZERO_EINVAL;
    if (nonfinite_flag != nullptr && (const void *)nonfinite_flag == (const void *)skip_if_nonzero)
        return ZERO_EINVAL;
    AdamConsts c;
    int rc = adam_consts(hp, t, &c);
    if (rc != ZERO_OK)
        return rc;
    if (n_tensors > ZERO_NOALLOC_MAX_TENSORS)
        return ZERO_ERANGE;
    // the plan builder's classification and checks, on the stack
    TensorDesc d[ZERO_NOALLOC_MAX_TENSORS];
    zs::Range r[5 * ZERO_NOALLOC_MAX_TENSORS];
    size_t nd = 0;
    uint64_t n_params = 0;
    for (uint32_t k = 0; k < n_tensors; k++) {
        if (tensors[k].n == 0)
            continue;
        if ((rc = zs::describe_tensor(tensors[k], &d[nd], &r[5 * nd])) != ZERO_OK)
            return rc;
        if (__builtin_add_overflow(n_params, tensors[k].n, &n_params))
            return ZERO_EOVERFLOW;
        nd++;
    }
    if (zs::writes_overlap(r, 5 * nd))
        return ZERO_EINVAL;
    if (nd == 0)
        return ZERO_OK;
    const uint64_t C = zs::pick_chunk(d, nd);
    zero_plan_stats stats;
    zs::plan_stats(d, nd, n_tensors, C, &stats);
    if (stats.table_bytes > ZERO_NOALLOC_SCRATCH_BYTES)
        return ZERO_ERANGE;
    int dev = -1;
    if ((rc = current_device(&dev)) != ZERO_OK)
        return rc;
    unsigned char *table = nullptr;
    if ((rc = noalloc_table(dev, &table)) != ZERO_OK)
        return rc;
    TensorDesc *d_tensors = (TensorDesc *)table;
    Chunk *d_chunks = (Chunk *)(table + nd * sizeof(TensorDesc));
    hipStream_t st = (hipStream_t)stream;
    uint64_t c0 = 0;
    for (size_t b = 0; b < nd; b += kStageBatch) {
        const uint32_t count = (uint32_t)(nd - b < kStageBatch ? nd - b : kStageBatch);
        StageArgs a;
        memset(&a, 0, sizeof(a));
        for (uint32_t j = 0; j < count; j++) {
            a.d[j] = d[b + j];
            a.chunk0[j] = c0;
            c0 += zs::chunks_of(d[b + j], C);
        }
        a.chunk0[count] = c0;
        const uint64_t work = a.chunk0[count] - a.chunk0[0];
        const uint64_t want = ((work > count ? work : count) + 255) / 256;
        const uint32_t grid = (uint32_t)(want < 1024 ? want : 1024);
        hipLaunchKernelGGL(zs_stage_table_kernel, dim3(grid), dim3(256), 0, st, a, (uint32_t)b,
                           count, C, d_tensors, d_chunks);
        if (hipGetLastError() != hipSuccess)
            return ZERO_EHIP;
    }
    const size_t lds = lds_cap_bytes(dev, (uint32_t)stats.wg_per_cu);
    return launch_adam_table(d_tensors, d_chunks, stats, lds, false, zs::any_shift(d, nd), c,
                             nonfinite_flag, skip_if_nonzero, nullptr, st);
}
