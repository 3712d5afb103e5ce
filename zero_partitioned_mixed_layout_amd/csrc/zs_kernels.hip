// zs_kernels.hip -- the device side of libzeroshard.so for gfx950 (CDNA4):
// the fused multi-tensor Adam step and the N_d-slice gradient reduction, plus
// the plan upload and the launches behind the C ABI.
//
// Both kernels are elementwise HBM streams (Adam: 28 bytes per parameter;
// reduce: 2 N_d + 2 bytes), so they use no matrix cores.  Each lane moves
// 16-byte vectors (8 fp16 or 4 fp32), a 64-lane wave covers contiguous
// 1-2 KiB per instruction, and streamed data is loaded and stored with the
// nontemporal hint so it does not displace anything in the caches.
//
// Exactness: every arithmetic step is one IEEE binary32 operation in a fixed
// order; the library is built with -ffp-contract=off (no fused multiply-add),
// fp32 denormals kept, and correctly rounded fp32 division and square root.
// fp16 <-> fp32 conversions are the hardware's (v_cvt_f32_f16 is exact,
// v_cvt_f16_f32 rounds to nearest even in the default mode).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>

#include "zero_shard.h"
#include "zs_internal.h"

namespace {

using zs::Chunk;
using zs::kBlock;
using zs::TensorDesc;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

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
};

template <typename T>
__device__ __forceinline__ T ld_nt(const T *p) {
    return __builtin_nontemporal_load(as_global(p));
}
template <typename T>
__device__ __forceinline__ void st_nt(T v, T *p) {
    __builtin_nontemporal_store(v, as_global(p));
}

__device__ __forceinline__ bool f16_bits_nonfinite(uint16_t b) {
    return (b & 0x7C00u) == 0x7C00u;
}

// One element of the Adam step (Kingma and Ba, Algorithm 1, with bias
// correction and eps outside the root).  Returns the new fp16 parameter.
__device__ __forceinline__ _Float16 adam_elem(float g, float &w, float &m, float &v,
                                              const AdamConsts &c) {
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
    return (_Float16)w;
}

__device__ __forceinline__ void adam_single(const TensorDesc &T, uint64_t i,
                                            const AdamConsts &c, int &bad) {
    const uint16_t gb = as_global(T.g)[i];
    bad |= f16_bits_nonfinite(gb);
    _Float16 gh;
    memcpy(&gh, &gb, 2);
    float w = as_global(T.w)[i], m = as_global(T.m)[i], v = as_global(T.v)[i];
    const _Float16 p = adam_elem((float)gh, w, m, v, c);
    as_global(T.w)[i] = w;
    as_global(T.m)[i] = m;
    as_global(T.v)[i] = v;
    uint16_t pb;
    memcpy(&pb, &p, 2);
    as_global(T.p)[i] = pb;
}

// 8 consecutive elements from a 16-byte-aligned group start i.
__device__ __forceinline__ void adam_vec8(const TensorDesc &T, uint64_t i,
                                          const AdamConsts &c, int &bad) {
    const f16x8 g = ld_nt(reinterpret_cast<const f16x8 *>(T.g + i));
    f32x4 w0 = ld_nt(reinterpret_cast<const f32x4 *>(T.w + i));
    f32x4 w1 = ld_nt(reinterpret_cast<const f32x4 *>(T.w + i + 4));
    f32x4 m0 = ld_nt(reinterpret_cast<const f32x4 *>(T.m + i));
    f32x4 m1 = ld_nt(reinterpret_cast<const f32x4 *>(T.m + i + 4));
    f32x4 v0 = ld_nt(reinterpret_cast<const f32x4 *>(T.v + i));
    f32x4 v1 = ld_nt(reinterpret_cast<const f32x4 *>(T.v + i + 4));
    // keep all seven 16-byte loads in flight before any arithmetic
    __builtin_amdgcn_sched_barrier(0);
    f16x8 p;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        uint16_t gb;
        _Float16 gj = g[j];
        memcpy(&gb, &gj, 2);
        bad |= f16_bits_nonfinite(gb);
        float w = w0[j], m = m0[j], v = v0[j];
        p[j] = adam_elem((float)gj, w, m, v, c);
        w0[j] = w;
        m0[j] = m;
        v0[j] = v;
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
        uint16_t gb;
        _Float16 gj = g[j + 4];
        memcpy(&gb, &gj, 2);
        bad |= f16_bits_nonfinite(gb);
        float w = w1[j], m = m1[j], v = v1[j];
        p[j + 4] = adam_elem((float)gj, w, m, v, c);
        w1[j] = w;
        m1[j] = m;
        v1[j] = v;
    }
    st_nt(w0, reinterpret_cast<f32x4 *>(T.w + i));
    st_nt(w1, reinterpret_cast<f32x4 *>(T.w + i + 4));
    st_nt(m0, reinterpret_cast<f32x4 *>(T.m + i));
    st_nt(m1, reinterpret_cast<f32x4 *>(T.m + i + 4));
    st_nt(v0, reinterpret_cast<f32x4 *>(T.v + i));
    st_nt(v1, reinterpret_cast<f32x4 *>(T.v + i + 4));
    st_nt(p, reinterpret_cast<f16x8 *>(T.p + i));
}

// 4 consecutive elements: fp16 arrays 8-byte aligned, fp32 16-byte aligned.
__device__ __forceinline__ void adam_vec4(const TensorDesc &T, uint64_t i,
                                          const AdamConsts &c, int &bad) {
    const f16x4 g = ld_nt(reinterpret_cast<const f16x4 *>(T.g + i));
    f32x4 w0 = ld_nt(reinterpret_cast<const f32x4 *>(T.w + i));
    f32x4 m0 = ld_nt(reinterpret_cast<const f32x4 *>(T.m + i));
    f32x4 v0 = ld_nt(reinterpret_cast<const f32x4 *>(T.v + i));
    __builtin_amdgcn_sched_barrier(0);
    f16x4 p;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        uint16_t gb;
        _Float16 gj = g[j];
        memcpy(&gb, &gj, 2);
        bad |= f16_bits_nonfinite(gb);
        float w = w0[j], m = m0[j], v = v0[j];
        p[j] = adam_elem((float)gj, w, m, v, c);
        w0[j] = w;
        m0[j] = m;
        v0[j] = v;
    }
    st_nt(w0, reinterpret_cast<f32x4 *>(T.w + i));
    st_nt(m0, reinterpret_cast<f32x4 *>(T.m + i));
    st_nt(v0, reinterpret_cast<f32x4 *>(T.v + i));
    st_nt(p, reinterpret_cast<f16x4 *>(T.p + i));
}

template <int VEC>
__device__ __forceinline__ void adam_chunk(const TensorDesc &T, const Chunk &ch,
                                           const AdamConsts &c, int &bad) {
    const uint32_t tid = threadIdx.x;
    // the tensor's unaligned head belongs to its first chunk
    const uint32_t head = ch.start == 0 ? min(T.head, ch.count) : 0u;
    if (tid < head)
        adam_single(T, ch.start + tid, c, bad);
    const uint64_t base = ch.start + head;
    const uint32_t nvec = (ch.count - head) / VEC;
    for (uint32_t k = tid; k < nvec; k += kBlock) {
        if (VEC == 8)
            adam_vec8(T, base + (uint64_t)k * 8, c, bad);
        else
            adam_vec4(T, base + (uint64_t)k * 4, c, bad);
    }
    const uint64_t tail0 = base + (uint64_t)nvec * VEC;
    const uint32_t tail = ch.count - head - nvec * VEC;
    if (tid < tail)
        adam_single(T, tail0 + tid, c, bad);
}

__global__ __launch_bounds__(kBlock) void zs_adam_kernel(
    const TensorDesc *__restrict__ tensors, const Chunk *__restrict__ chunks,
    uint64_t n_chunks, AdamConsts c, int32_t *__restrict__ flag,
    const int32_t *__restrict__ skip) {
    if (skip != nullptr && *skip != 0)
        return; // the same value for every wave: the whole step is skipped
    int bad = 0;
    for (uint64_t ci = blockIdx.x; ci < n_chunks; ci += gridDim.x) {
        const Chunk ch = chunks[ci];
        const TensorDesc T = tensors[ch.tensor];
        if (T.vec == 8) {
            adam_chunk<8>(T, ch, c, bad);
        } else if (T.vec == 4) {
            adam_chunk<4>(T, ch, c, bad);
        } else {
            for (uint32_t k = threadIdx.x; k < ch.count; k += kBlock)
                adam_single(T, ch.start + k, c, bad);
        }
    }
    // one atomic per wave at most, and only from a wave that saw a
    // non-finite gradient anywhere in its share of the grid-stride loop
    if (flag != nullptr) {
        const uint64_t any = __ballot(bad);
        if (any != 0 && (threadIdx.x & 63) == 0)
            atomicOr(flag, 1);
    }
}

// ---------------------------------------------------------------------------
// Gradient reduction over N_d slices.
// ---------------------------------------------------------------------------
struct SliceArgs {
    const _Float16 *p[ZERO_MAX_SLICES];
};

__device__ __forceinline__ float reduce_single(const SliceArgs &s, uint32_t nd, uint64_t i) {
    float acc = (float)as_global(s.p[0])[i];
    for (uint32_t r = 1; r < nd; r++)
        acc = acc + (float)as_global(s.p[r])[i];
    return acc;
}

template <int VEC>
struct HVec;
template <>
struct HVec<8> {
    typedef f16x8 T;
};
template <>
struct HVec<4> {
    typedef f16x4 T;
};

template <int VEC>
__device__ __forceinline__ void reduce_group(const SliceArgs &s, uint32_t nd, uint64_t i,
                                             float count, _Float16 *out, int &bad) {
    typedef typename HVec<VEC>::T hv;
    constexpr int B = 8; // slices in flight per lane
    float acc[VEC];
    uint32_t r;
    if (nd >= B) {
        hv x[B];
#pragma unroll
        for (int q = 0; q < B; q++)
            x[q] = ld_nt(reinterpret_cast<const hv *>(s.p[q] + i));
        // all loads in flight before the first add
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < VEC; j++)
            acc[j] = (float)x[0][j];
#pragma unroll
        for (int q = 1; q < B; q++)
#pragma unroll
            for (int j = 0; j < VEC; j++)
                acc[j] = acc[j] + (float)x[q][j];
        r = B;
    } else {
        const hv x = ld_nt(reinterpret_cast<const hv *>(s.p[0] + i));
#pragma unroll
        for (int j = 0; j < VEC; j++)
            acc[j] = (float)x[j];
        r = 1;
    }
    // the sums stay in rank order: slice r is added after slices 0..r-1
    for (; r + B <= nd; r += B) {
        hv x[B];
#pragma unroll
        for (int q = 0; q < B; q++)
            x[q] = ld_nt(reinterpret_cast<const hv *>(s.p[r + q] + i));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < B; q++)
#pragma unroll
            for (int j = 0; j < VEC; j++)
                acc[j] = acc[j] + (float)x[q][j];
    }
    for (; r < nd; r++) {
        const hv x = ld_nt(reinterpret_cast<const hv *>(s.p[r] + i));
#pragma unroll
        for (int j = 0; j < VEC; j++)
            acc[j] = acc[j] + (float)x[j];
    }
    hv o;
#pragma unroll
    for (int j = 0; j < VEC; j++) {
        o[j] = (_Float16)(acc[j] / count);
        uint16_t b;
        _Float16 oj = o[j];
        memcpy(&b, &oj, 2);
        bad |= f16_bits_nonfinite(b);
    }
    st_nt(o, reinterpret_cast<hv *>(out + i));
}

template <int VEC>
__global__ __launch_bounds__(kBlock) void zs_reduce_kernel(SliceArgs s, uint32_t nd, uint64_t n,
                                                           uint32_t head, _Float16 *__restrict__ out,
                                                           int32_t *__restrict__ flag) {
    const float count = (float)nd;
    const uint64_t gtid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t gstride = (uint64_t)gridDim.x * kBlock;
    int bad = 0;
    const uint64_t h = head < n ? head : n;
    const uint64_t ngroups = VEC > 1 ? (n - h) / VEC : 0;
    const uint64_t body_end = h + ngroups * VEC;
    // unaligned head and tail, one element per thread
    if (gtid < h) {
        const _Float16 o = (_Float16)(reduce_single(s, nd, gtid) / count);
        as_global(out)[gtid] = o;
        uint16_t b;
        memcpy(&b, &o, 2);
        bad |= f16_bits_nonfinite(b);
    }
    for (uint64_t i = body_end + gtid; i < n; i += gstride) {
        const _Float16 o = (_Float16)(reduce_single(s, nd, i) / count);
        as_global(out)[i] = o;
        uint16_t b;
        memcpy(&b, &o, 2);
        bad |= f16_bits_nonfinite(b);
    }
    if (VEC > 1)
        for (uint64_t k = gtid; k < ngroups; k += gstride)
            reduce_group<VEC == 8 ? 8 : 4>(s, nd, h + k * VEC, count, out, bad);
    if (flag != nullptr) {
        const uint64_t any = __ballot(bad);
        if (any != 0 && (threadIdx.x & 63) == 0)
            atomicOr(flag, 1);
    }
}

// Workgroups of a grid-stride launch: enough to give each of the 256 CUs
// several resident workgroups, never more than the work needs.
uint32_t grid_for(uint64_t items_per_thread_units, uint32_t cap) {
    const uint64_t want = (items_per_thread_units + kBlock - 1) / kBlock;
    return (uint32_t)(want < 1 ? 1 : (want > cap ? cap : want));
}

} // namespace

struct zero_plan {
    zs::TensorDesc *d_tensors;
    zs::Chunk *d_chunks;
    void *d_table;
    zero_plan_stats stats;
    int device;
};

extern "C" int zero_plan_create(const zero_tensor *tensors, uint32_t n_tensors, zero_plan **out) {
    if (!out)
        return ZERO_EINVAL;
    zs::HostPlan hp;
    int rc = zs::build_host_plan(tensors, n_tensors, &hp);
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

extern "C" int zero_adam_step(const zero_plan *plan, const zero_adam_hparams *hp, uint64_t t,
                              int32_t *nonfinite_flag, const int32_t *skip_if_nonzero,
                              void *stream) {
    if (!plan || !hp)
        return ZERO_EINVAL;
    if (nonfinite_flag != nullptr && (const void *)nonfinite_flag == (const void *)skip_if_nonzero)
        return ZERO_EINVAL;
    float s[8];
    int rc = zero_adam_scalars(hp, t, s);
    if (rc != ZERO_OK)
        return rc;
    if (plan->stats.n_chunks == 0)
        return ZERO_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return ZERO_EHIP;
    }
    if (dev != plan->device)
        return ZERO_EINVAL;
    const AdamConsts c = {s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]};
    // one workgroup per chunk, up to 16 resident per CU on 256 CUs; larger
    // plans grid-stride
    const uint64_t nch = plan->stats.n_chunks;
    const uint32_t grid = (uint32_t)(nch < 256u * 16u ? nch : 256u * 16u);
    hipLaunchKernelGGL(zs_adam_kernel, dim3(grid), dim3(kBlock), 0, (hipStream_t)stream,
                       plan->d_tensors, plan->d_chunks, nch, c, nonfinite_flag, skip_if_nonzero);
    if (hipGetLastError() != hipSuccess)
        return ZERO_EHIP;
    return ZERO_OK;
}

extern "C" int zero_reduce_grad_shard(const void *const *slices_f16, uint32_t nd, uint64_t n,
                                      void *out_f16, int32_t *nonfinite_flag, void *stream) {
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
        args.p[r] = (const _Float16 *)slices_f16[r];
        addr[r] = a;
    }
    for (uint32_t r = nd; r < ZERO_MAX_SLICES; r++)
        args.p[r] = nullptr;
    if (n == 0)
        return ZERO_OK;
    addr[nd] = o;
    uint32_t vec, head;
    zs::pick_vector_path(addr, (int)nd + 1, nullptr, 0, &vec, &head);
    const uint64_t groups = vec > 1 ? (n - (head < n ? head : n)) / vec + 1 : n;
    const uint32_t grid = grid_for(groups, 256u * 32u);
    hipStream_t st = (hipStream_t)stream;
    if (vec == 8)
        hipLaunchKernelGGL(zs_reduce_kernel<8>, dim3(grid), dim3(kBlock), 0, st, args, nd, n,
                           head, (_Float16 *)out_f16, nonfinite_flag);
    else if (vec == 4)
        hipLaunchKernelGGL(zs_reduce_kernel<4>, dim3(grid), dim3(kBlock), 0, st, args, nd, n,
                           head, (_Float16 *)out_f16, nonfinite_flag);
    else
        hipLaunchKernelGGL(zs_reduce_kernel<1>, dim3(grid), dim3(kBlock), 0, st, args, nd, n,
                           0u, (_Float16 *)out_f16, nonfinite_flag);
    if (hipGetLastError() != hipSuccess)
        return ZERO_EHIP;
    return ZERO_OK;
}
