// zs_offload.cpp -- the ZeRO-Offload variant of the shard step.  The fp32
// master, momentum and variance live in host memory and the host CPU runs
// the Adam update; the GPU keeps the fp16 parameters and gradients, and only
// those cross PCIe: the gradient shard to the host, the fresh fp16
// parameters back ([ER10] "The Breakthrough" and "The Mathematics", the
// paragraph on ZeRO-Offload; [DSZ] "Offload trades capacity against
// movement").
//
// The CPU update does, per element, the same IEEE binary32 operations in the
// same order as the GPU kernel (no fused multiply-add: the vector code is
// AVX2 without FMA, built with -ffp-contract=off), with F16C conversions
// (exact widening; narrowing rounds to nearest even), so host and device
// results are bit-identical.  The GPU entry points never call it.
//
// zero_offload_step pipelines the shard in chunks through three pinned
// staging slots: while the CPU threads update chunk k, the copy engines move
// chunk k+1's gradients in and chunk k-1's parameters out, on two streams of
// their own (default priority).
#include <hip/hip_runtime.h>
#include <immintrin.h>
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "zero_shard.h"
#include "zs_internal.h"

namespace {

struct HostConsts {
    float lr, b1, omb1, b2, omb2, bc1, bc2, eps;
};

bool cpu_has_avx2_f16c() {
    return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("f16c");
}

// The 16-bit formats of parameters and gradients, as on the device: IEEE
// binary16 (F16C conversions) and bfloat16 (widening is a 16-bit shift;
// narrowing rounds to nearest even in integer arithmetic, and a NaN stays a
// quiet NaN with its sign).  A value is infinite or NaN when its exponent
// field is all ones.
struct HostF16 {
    static constexpr uint16_t kExp = 0x7C00;
};
struct HostBF16 {
    static constexpr uint16_t kExp = 0x7F80;
};

#define ZS_HOST_SIMD __attribute__((target("avx2,f16c")))

ZS_HOST_SIMD inline float widen1(HostF16, uint16_t b) { return _cvtsh_ss(b); }
ZS_HOST_SIMD inline uint16_t narrow1(HostF16, float x) {
    return _cvtss_sh(x, _MM_FROUND_TO_NEAREST_INT);
}
ZS_HOST_SIMD inline __m256 widen8(HostF16, __m128i h) { return _mm256_cvtph_ps(h); }
ZS_HOST_SIMD inline __m128i narrow8(HostF16, __m256 x) {
    return _mm256_cvtps_ph(x, _MM_FROUND_TO_NEAREST_INT);
}

ZS_HOST_SIMD inline float widen1(HostBF16, uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return x;
}
ZS_HOST_SIMD inline uint16_t narrow1(HostBF16, float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
ZS_HOST_SIMD inline __m256 widen8(HostBF16, __m128i h) {
    return _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
}
ZS_HOST_SIMD inline __m128i narrow8(HostBF16, __m256 x) {
    const __m256i u = _mm256_castps_si256(x);
    const __m256i hi = _mm256_srli_epi32(u, 16);
    const __m256i lsb = _mm256_and_si256(hi, _mm256_set1_epi32(1));
    __m256i r = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(u, _mm256_set1_epi32(0x7FFF)),
                                                   lsb), 16);
    const __m256i qnan = _mm256_or_si256(hi, _mm256_set1_epi32(0x0040));
    r = _mm256_blendv_epi8(r, qnan, _mm256_castps_si256(_mm256_cmp_ps(x, x, _CMP_UNORD_Q)));
    // eight 32-bit values below 2^16 to eight 16-bit ones, in order
    const __m256i packed = _mm256_packus_epi32(r, r);
    return _mm256_castsi256_si128(_mm256_permute4x64_epi64(packed, 0x08));
}

// One element: the Adam step of Kingma and Ba's Algorithm 1 with bias
// correction, eps outside the root, in the GPU kernel's operation order.
template <class Fmt>
ZS_HOST_SIMD inline uint16_t adam_elem_host(uint16_t gb, float &w, float &m, float &v,
                                            const HostConsts &c) {
    const float g = widen1(Fmt(), gb);
    const float m_old = c.b1 * m;
    const float m_in = c.omb1 * g;
    m = m_old + m_in;
    const float v_old = c.b2 * v;
    const float g2 = g * g;
    const float v_in = c.omb2 * g2;
    v = v_old + v_in;
    const float m_hat = m / c.bc1;
    const float v_hat = v / c.bc2;
    const float root = _mm_cvtss_f32(_mm_sqrt_ss(_mm_set_ss(v_hat)));
    const float denom = root + c.eps;
    const float u = m_hat / denom;
    const float step = c.lr * u;
    w = w - step;
    return narrow1(Fmt(), w);
}

// Elements [0, n) of one range, eight at a time, then singly.  Returns 1 if
// any gradient is infinite or NaN.
template <class Fmt>
ZS_HOST_SIMD int adam_range_host(const uint16_t *g16, uint16_t *p16, float *w, float *m,
                                 float *v, uint64_t n, const HostConsts &c) {
    const __m256 lr = _mm256_set1_ps(c.lr), b1 = _mm256_set1_ps(c.b1),
                 omb1 = _mm256_set1_ps(c.omb1), b2 = _mm256_set1_ps(c.b2),
                 omb2 = _mm256_set1_ps(c.omb2), bc1 = _mm256_set1_ps(c.bc1),
                 bc2 = _mm256_set1_ps(c.bc2), eps = _mm256_set1_ps(c.eps);
    const __m128i expo = _mm_set1_epi16((short)Fmt::kExp);
    int bad = 0;
    uint64_t i = 0;
    // The 16-bit parameters are written only: streamed past the caches when
    // 16-byte aligned (no read for ownership of their lines; in the offload
    // pipeline the staging slot is read next by the copy engine, not the CPU).
    const bool p_aligned = ((uintptr_t)p16 & 15) == 0;
    for (; i + 8 <= n; i += 8) {
        const __m128i gh = _mm_loadu_si128(reinterpret_cast<const __m128i *>(g16 + i));
        bad |= _mm_movemask_epi8(_mm_cmpeq_epi16(_mm_and_si128(gh, expo), expo));
        const __m256 g = widen8(Fmt(), gh);
        const __m256 m_new = _mm256_add_ps(_mm256_mul_ps(b1, _mm256_loadu_ps(m + i)),
                                           _mm256_mul_ps(omb1, g));
        const __m256 v_new = _mm256_add_ps(_mm256_mul_ps(b2, _mm256_loadu_ps(v + i)),
                                           _mm256_mul_ps(omb2, _mm256_mul_ps(g, g)));
        const __m256 m_hat = _mm256_div_ps(m_new, bc1);
        const __m256 v_hat = _mm256_div_ps(v_new, bc2);
        const __m256 denom = _mm256_add_ps(_mm256_sqrt_ps(v_hat), eps);
        const __m256 step = _mm256_mul_ps(lr, _mm256_div_ps(m_hat, denom));
        const __m256 w_new = _mm256_sub_ps(_mm256_loadu_ps(w + i), step);
        _mm256_storeu_ps(m + i, m_new);
        _mm256_storeu_ps(v + i, v_new);
        _mm256_storeu_ps(w + i, w_new);
        const __m128i ph = narrow8(Fmt(), w_new);
        if (p_aligned)
            _mm_stream_si128(reinterpret_cast<__m128i *>(p16 + i), ph);
        else
            _mm_storeu_si128(reinterpret_cast<__m128i *>(p16 + i), ph);
    }
    _mm_sfence(); // the streamed parameters are visible before this range returns
    for (; i < n; i++) {
        bad |= (g16[i] & Fmt::kExp) == Fmt::kExp;
        p16[i] = adam_elem_host<Fmt>(g16[i], w[i], m[i], v[i], c);
    }
    return bad != 0;
}

// Most host threads an update may use.
constexpr uint32_t kMaxHostThreads = 1024;

// A fixed set of worker threads; run(f) calls f(0..parts-1) with the calling
// thread taking part 0 and returns when every part is done.  If a thread
// cannot start, the ones already started are stopped and joined before the
// exception leaves the constructor.
class Pool {
public:
    // cpus: NULL, or the CPUs every worker thread (not the caller's) is
    // pinned to when it starts.
    explicit Pool(uint32_t parts, const cpu_set_t *cpus = nullptr) : parts_(parts) {
        if (cpus)
            cpus_ = *cpus;
        const bool pin = cpus != nullptr;
        try {
            for (uint32_t k = 1; k < parts; k++)
                threads_.emplace_back([this, k, pin] {
                    if (pin)
                        (void)pthread_setaffinity_np(pthread_self(), sizeof(cpus_), &cpus_);
                    work(k);
                });
        } catch (...) {
            shutdown();
            throw;
        }
    }
    ~Pool() { shutdown(); }
    uint32_t parts() const { return parts_; }
    void run(const std::function<void(uint32_t)> &f) {
        {
            std::lock_guard<std::mutex> lk(mu_);
            job_ = &f;
            pending_ = parts_ - 1;
            gen_++;
        }
        cv_.notify_all();
        f(0);
        std::unique_lock<std::mutex> lk(mu_);
        done_.wait(lk, [this] { return pending_ == 0; });
        job_ = nullptr;
    }

private:
    void shutdown() {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (std::thread &t : threads_)
            if (t.joinable())
                t.join();
        threads_.clear();
    }
    void work(uint32_t k) {
        uint64_t seen = 0;
        for (;;) {
            std::unique_lock<std::mutex> lk(mu_);
            cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
            if (stop_)
                return;
            seen = gen_;
            const std::function<void(uint32_t)> *f = job_;
            lk.unlock();
            (*f)(k);
            lk.lock();
            if (--pending_ == 0)
                done_.notify_one();
        }
    }
    uint32_t parts_;
    cpu_set_t cpus_;
    std::vector<std::thread> threads_;
    std::mutex mu_;
    std::condition_variable cv_, done_;
    const std::function<void(uint32_t)> *job_ = nullptr;
    uint32_t pending_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

// The update of n elements split over the pool's parts in contiguous ranges
// of whole groups of eight.  Returns 1 if any gradient is non-finite.
template <class Fmt>
int adam_parallel(Pool &pool, const uint16_t *g16, uint16_t *p16, float *w, float *m, float *v,
                  uint64_t n, const HostConsts &c) {
    const uint32_t P = pool.parts();
    std::vector<int> bad(P, 0);
    const uint64_t groups = (n + 7) / 8;
    pool.run([&](uint32_t k) {
        const uint64_t lo = std::min(n, groups * k / P * 8);
        const uint64_t hi = std::min(n, groups * (k + 1) / P * 8);
        if (hi > lo)
            bad[k] = adam_range_host<Fmt>(g16 + lo, p16 + lo, w + lo, m + lo, v + lo, hi - lo,
                                          c);
    });
    int any = 0;
    for (int b : bad)
        any |= b;
    return any;
}

// The CPUs this process may run on.
uint32_t affinity_count() {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0 && CPU_COUNT(&set) > 0)
        return (uint32_t)CPU_COUNT(&set);
    const unsigned hw = std::thread::hardware_concurrency();
    return hw == 0 ? 1u : hw;
}

// Host threads of an update when the caller leaves it to the library: the
// CPUs available (`cpus`, or the process's), at most 16.  The host update
// is bound by host memory bandwidth, which 16 threads already drive (the
// measurements behind this are in the build's design notes).
uint32_t default_threads(uint32_t cpus = 0) {
    return std::min(16u, cpus ? cpus : affinity_count());
}

// The NUMA node of device `dev` as the host's sysfs reports it (-1 if
// unknown), and in *set the CPUs of that node this process may run on.
// Returns how many there are (0: no placement to make).
uint32_t gpu_node_cpus(int dev, int *node, cpu_set_t *set) {
    *node = -1;
    CPU_ZERO(set);
    char bus[64] = {0};
    if (hipDeviceGetPCIBusId(bus, (int)sizeof(bus) - 1, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    for (char *c = bus; *c; c++)
        if (*c >= 'A' && *c <= 'F')
            *c = (char)(*c - 'A' + 'a');
    char path[256];
    snprintf(path, sizeof(path), "/sys/bus/pci/devices/%s/numa_node", bus);
    FILE *f = fopen(path, "r");
    if (!f)
        return 0;
    const int got = fscanf(f, "%d", node);
    fclose(f);
    if (got != 1 || *node < 0) {
        *node = -1;
        return 0;
    }
    snprintf(path, sizeof(path), "/sys/devices/system/node/node%d/cpulist", *node);
    f = fopen(path, "r");
    if (!f)
        return 0;
    // "a-b,c,d-e": ranges of CPU numbers
    cpu_set_t node_cpus;
    CPU_ZERO(&node_cpus);
    int lo, hi;
    char sep;
    while (fscanf(f, "%d", &lo) == 1) {
        hi = lo;
        sep = (char)fgetc(f);
        if (sep == '-') {
            if (fscanf(f, "%d", &hi) != 1)
                break;
            sep = (char)fgetc(f);
        }
        for (int c = lo; c <= hi && c < CPU_SETSIZE; c++)
            if (c >= 0)
                CPU_SET(c, &node_cpus);
        if (sep != ',')
            break;
    }
    fclose(f);
    cpu_set_t mine;
    if (sched_getaffinity(0, sizeof(mine), &mine) != 0)
        return 0;
    CPU_AND(set, &node_cpus, &mine);
    return (uint32_t)CPU_COUNT(set);
}

// Host arrays: non-null when n > 0, aligned to their element size, the
// written ones overlapping nothing.
int check_host_arrays(const void *grad, const void *param, const float *w, const float *m,
                      const float *v, uint64_t n) {
    uint64_t b2, b4;
    if (__builtin_mul_overflow(n, (uint64_t)2, &b2) || __builtin_mul_overflow(n, (uint64_t)4, &b4))
        return ZERO_EOVERFLOW;
    if (n == 0)
        return ZERO_OK;
    const uintptr_t g = (uintptr_t)grad, p = (uintptr_t)param, a = (uintptr_t)w,
                    b = (uintptr_t)m, d = (uintptr_t)v;
    if (!g || !p || !a || !b || !d || (g | p) % 2 || (a | b | d) % 4)
        return ZERO_EINVAL;
    std::vector<zs::Range> r = {{g, g + b2, false}, {p, p + b2, true}, {a, a + b4, true},
                                {b, b + b4, true}, {d, d + b4, true}};
    for (const zs::Range &x : r)
        if (x.hi < x.lo)
            return ZERO_EOVERFLOW;
    return zs::writes_overlap(r) ? ZERO_EINVAL : ZERO_OK;
}

template <class Fmt>
int adam_step_host(const void *grad_f16, void *param_f16, float *master, float *m, float *v,
                   uint64_t n, const zero_adam_hparams *hp, uint64_t t, uint32_t threads,
                   int32_t *nonfinite_flag) {
    if (!hp)
        return ZERO_EINVAL;
    float s[8];
    int rc = zero_adam_scalars(hp, t, s);
    if (rc != ZERO_OK)
        return rc;
    if (threads > kMaxHostThreads)
        return ZERO_EINVAL;
    rc = check_host_arrays(grad_f16, param_f16, master, m, v, n);
    if (rc != ZERO_OK)
        return rc;
    if (!cpu_has_avx2_f16c())
        return ZERO_ENOTSUP;
    if (n == 0)
        return ZERO_OK;
    const HostConsts c = {s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]};
    try {
        Pool pool(threads ? threads : default_threads());
        const int bad = adam_parallel<Fmt>(pool, (const uint16_t *)grad_f16,
                                           (uint16_t *)param_f16, master, m, v, n, c);
        if (bad && nonfinite_flag)
            *nonfinite_flag |= 1;
    } catch (...) {
        return ZERO_ENOMEM;
    }
    return ZERO_OK;
}

} // namespace

extern "C" int zero_adam_step_host(const void *grad_f16, void *param_f16, float *master, float *m,
                                   float *v, uint64_t n, const zero_adam_hparams *hp, uint64_t t,
                                   uint32_t threads, int32_t *nonfinite_flag) {
    return adam_step_host<HostF16>(grad_f16, param_f16, master, m, v, n, hp, t, threads,
                                   nonfinite_flag);
}

extern "C" int zero_adam_step_host_bf16(const void *grad_bf16, void *param_bf16, float *master,
                                        float *m, float *v, uint64_t n,
                                        const zero_adam_hparams *hp, uint64_t t,
                                        uint32_t threads, int32_t *nonfinite_flag) {
    return adam_step_host<HostBF16>(grad_bf16, param_bf16, master, m, v, n, hp, t, threads,
                                    nonfinite_flag);
}

// ---------------------------------------------------------------------------
// The offload pipeline.
// ---------------------------------------------------------------------------
struct zero_offload {
    static constexpr int kSlots = 3;
    int device = 0;
    uint64_t chunk = 0;
    Pool *pool = nullptr;
    zero_offload_info info = {};
    hipStream_t d2h = nullptr, h2d = nullptr;
    hipEvent_t ready = nullptr;
    hipEvent_t d2h_done[kSlots] = {};
    hipEvent_t h2d_done[kSlots] = {};
    uint16_t *g_stage[kSlots] = {};
    uint16_t *p_stage[kSlots] = {};
};

namespace {

void offload_free(zero_offload *o) {
    if (!o)
        return;
    for (int k = 0; k < zero_offload::kSlots; k++) {
        if (o->g_stage[k])
            (void)hipHostFree(o->g_stage[k]);
        if (o->p_stage[k])
            (void)hipHostFree(o->p_stage[k]);
        if (o->d2h_done[k])
            (void)hipEventDestroy(o->d2h_done[k]);
        if (o->h2d_done[k])
            (void)hipEventDestroy(o->h2d_done[k]);
    }
    if (o->ready)
        (void)hipEventDestroy(o->ready);
    if (o->d2h)
        (void)hipStreamDestroy(o->d2h);
    if (o->h2d)
        (void)hipStreamDestroy(o->h2d);
    delete o->pool;
    (void)hipGetLastError();
    delete o;
}

} // namespace

extern "C" int zero_offload_create(uint64_t chunk_elems, uint32_t threads, zero_offload **out) {
    if (!out)
        return ZERO_EINVAL;
    if (chunk_elems == 0)
        chunk_elems = zs::kOffloadChunk;
    if (chunk_elems % 8 != 0 || chunk_elems > (1ull << 32) || threads > kMaxHostThreads)
        return ZERO_EINVAL;
    if (!cpu_has_avx2_f16c())
        return ZERO_ENOTSUP;
    zero_offload *o = new (std::nothrow) zero_offload;
    if (!o)
        return ZERO_ENOMEM;
    o->chunk = chunk_elems;
    if (hipGetDevice(&o->device) != hipSuccess) {
        offload_free(o);
        return ZERO_EHIP;
    }
    // the update's threads go to the GPU's NUMA node when the host says
    // which it is (the caller first-touches the fp32 state there)
    int node = -1;
    cpu_set_t node_cpus;
    const uint32_t n_node = gpu_node_cpus(o->device, &node, &node_cpus);
    const uint32_t nthreads = threads ? threads : default_threads(n_node);
    try {
        o->pool = new Pool(nthreads, n_node ? &node_cpus : nullptr);
    } catch (...) {
        offload_free(o);
        return ZERO_ENOMEM;
    }
    o->info.threads = nthreads;
    o->info.numa_node = node;
    o->info.pinned_cpus = n_node;
    o->info.chunk_elems = chunk_elems;
    bool ok = hipStreamCreateWithFlags(&o->d2h, hipStreamNonBlocking) == hipSuccess &&
              hipStreamCreateWithFlags(&o->h2d, hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&o->ready, hipEventDisableTiming) == hipSuccess;
    for (int k = 0; ok && k < zero_offload::kSlots; k++)
        ok = hipEventCreateWithFlags(&o->d2h_done[k], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&o->h2d_done[k], hipEventDisableTiming) == hipSuccess;
    if (!ok) {
        offload_free(o);
        return ZERO_EHIP;
    }
    for (int k = 0; k < zero_offload::kSlots; k++) {
        if (hipHostMalloc((void **)&o->g_stage[k], chunk_elems * 2, hipHostMallocDefault) !=
                hipSuccess ||
            hipHostMalloc((void **)&o->p_stage[k], chunk_elems * 2, hipHostMallocDefault) !=
                hipSuccess) {
            offload_free(o);
            return ZERO_ENOMEM;
        }
    }
    *out = o;
    return ZERO_OK;
}

extern "C" int zero_offload_describe(const zero_offload *o, zero_offload_info *out) {
    if (!o || !out)
        return ZERO_EINVAL;
    *out = o->info;
    return ZERO_OK;
}

extern "C" int zero_offload_destroy(zero_offload *o) {
    if (!o)
        return ZERO_OK;
    int rc = ZERO_OK;
    if (hipStreamSynchronize(o->d2h) != hipSuccess || hipStreamSynchronize(o->h2d) != hipSuccess)
        rc = ZERO_EHIP;
    offload_free(o);
    return rc;
}

namespace {

template <class Fmt>
int offload_step(zero_offload *o, const void *grad_f16, void *param_f16, float *master, float *m,
                 float *v, uint64_t n, const zero_adam_hparams *hp, uint64_t t,
                 int32_t *nonfinite_flag, void *stream) {
    if (!o || !hp)
        return ZERO_EINVAL;
    float s[8];
    int rc = zero_adam_scalars(hp, t, s);
    if (rc != ZERO_OK)
        return rc;
    // grad and param are device arrays, master/m/v host arrays: two address
    // spaces, so overlaps are checked within each
    uint64_t b2, b4;
    if (__builtin_mul_overflow(n, (uint64_t)2, &b2) || __builtin_mul_overflow(n, (uint64_t)4, &b4))
        return ZERO_EOVERFLOW;
    if (n == 0)
        return ZERO_OK;
    const uintptr_t g = (uintptr_t)grad_f16, p = (uintptr_t)param_f16;
    if (!g || !p || (g | p) % 2 || g + b2 < g || p + b2 < p || (g < p + b2 && p < g + b2))
        return ZERO_EINVAL;
    {
        const uintptr_t a = (uintptr_t)master, b = (uintptr_t)m, d = (uintptr_t)v;
        if (!a || !b || !d || (a | b | d) % 4)
            return ZERO_EINVAL;
        std::vector<zs::Range> r = {{a, a + b4, true}, {b, b + b4, true}, {d, d + b4, true}};
        for (const zs::Range &x : r)
            if (x.hi < x.lo)
                return ZERO_EOVERFLOW;
        if (zs::writes_overlap(r))
            return ZERO_EINVAL;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return ZERO_EHIP;
    }
    if (dev != o->device)
        return ZERO_EINVAL;
    const HostConsts c = {s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]};
    const int S = zero_offload::kSlots;
    const uint64_t C = o->chunk;
    const uint64_t K = (n + C - 1) / C;
    const uint16_t *gd = (const uint16_t *)grad_f16;
    uint16_t *pd = (uint16_t *)param_f16;
    bool ok = true;
    auto count = [&](uint64_t k) { return std::min(C, n - k * C); };
    auto d2h = [&](uint64_t k) {
        const int slot = (int)(k % S);
        ok = ok && hipMemcpyAsync(o->g_stage[slot], gd + k * C, count(k) * 2,
                                  hipMemcpyDeviceToHost, o->d2h) == hipSuccess &&
             hipEventRecord(o->d2h_done[slot], o->d2h) == hipSuccess;
    };
    // the gradients are ready once the work already on `stream` is done
    ok = hipEventRecord(o->ready, (hipStream_t)stream) == hipSuccess &&
         hipStreamWaitEvent(o->d2h, o->ready, 0) == hipSuccess;
    for (uint64_t k = 0; k < K && k < (uint64_t)S; k++)
        d2h(k);
    int bad = 0;
    for (uint64_t k = 0; ok && k < K; k++) {
        const int slot = (int)(k % S);
        ok = hipEventSynchronize(o->d2h_done[slot]) == hipSuccess;
        if (ok && k >= (uint64_t)S) // the slot's previous parameters have left
            ok = hipEventSynchronize(o->h2d_done[slot]) == hipSuccess;
        if (!ok)
            break;
        try {
            bad |= adam_parallel<Fmt>(*o->pool, o->g_stage[slot], o->p_stage[slot], master + k * C,
                                 m + k * C, v + k * C, count(k), c);
        } catch (...) {
            ok = false;
            break;
        }
        ok = hipMemcpyAsync(pd + k * C, o->p_stage[slot], count(k) * 2, hipMemcpyHostToDevice,
                            o->h2d) == hipSuccess &&
             hipEventRecord(o->h2d_done[slot], o->h2d) == hipSuccess;
        if (k + S < K) // the CPU is done with this slot's gradients
            d2h(k + S);
    }
    // drain both copy streams before returning, also after an error
    const bool drained = hipStreamSynchronize(o->d2h) == hipSuccess &&
                         hipStreamSynchronize(o->h2d) == hipSuccess;
    if (!ok || !drained) {
        (void)hipGetLastError();
        return ZERO_EHIP;
    }
    if (bad && nonfinite_flag)
        *nonfinite_flag |= 1;
    return ZERO_OK;
}

} // namespace

extern "C" int zero_offload_step(zero_offload *o, const void *grad_f16, void *param_f16,
                                 float *master, float *m, float *v, uint64_t n,
                                 const zero_adam_hparams *hp, uint64_t t,
                                 int32_t *nonfinite_flag, void *stream) {
    return offload_step<HostF16>(o, grad_f16, param_f16, master, m, v, n, hp, t, nonfinite_flag,
                                 stream);
}

extern "C" int zero_offload_step_bf16(zero_offload *o, const void *grad_bf16, void *param_bf16,
                                      float *master, float *m, float *v, uint64_t n,
                                      const zero_adam_hparams *hp, uint64_t t,
                                      int32_t *nonfinite_flag, void *stream) {
    return offload_step<HostBF16>(o, grad_bf16, param_bf16, master, m, v, n, hp, t,
                                  nonfinite_flag, stream);
}
