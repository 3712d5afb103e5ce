// zs_host.cpp -- host-only logic of libzeroshard.so: shard layout, model-state
// ledger, Adam step constants, status strings and the multi-tensor plan
// builder.  Nothing here touches a device.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "zero_shard.h"
#include "zs_internal.h"

namespace {

// a * b + c with overflow detection, in 64-bit unsigned arithmetic.
bool mul_ok(uint64_t a, uint64_t b, uint64_t *r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(uint64_t a, uint64_t b, uint64_t *r) { return !__builtin_add_overflow(a, b, r); }

} // namespace

extern "C" int zero_shard_layout(uint64_t psi, uint32_t nd, uint32_t rank, uint32_t align,
                                 zero_layout *out) {
    if (!out || nd == 0 || align == 0 || rank >= nd)
        return ZERO_EINVAL;
    // Tail padding: round psi up to whole units of nd * align elements
    // ([16B] "The part that sounds too good: communication": each rank owns
    // one contiguous slice; the padding rule is this library's).
    const uint64_t unit = (uint64_t)nd * (uint64_t)align; // < 2^64: both < 2^32
    const uint64_t units = psi / unit + (psi % unit != 0);
    uint64_t padded;
    if (!mul_ok(units, unit, &padded))
        return ZERO_EOVERFLOW;
    const uint64_t shard = padded / nd;
    const uint64_t offset = (uint64_t)rank * shard; // <= padded
    out->padded_total = padded;
    out->shard_len = shard;
    out->offset = offset;
    out->real_len = offset >= psi ? 0 : std::min(shard, psi - offset);
    return ZERO_OK;
}

extern "C" int zero_state_bytes(uint32_t stage, uint64_t psi, uint32_t nd, uint32_t align,
                                uint64_t *out_bytes) {
    if (!out_bytes || stage > 3)
        return ZERO_EINVAL;
    zero_layout lay;
    int rc = zero_shard_layout(psi, nd, 0, align, &lay);
    if (rc != ZERO_OK)
        return rc;
    // [ER10] "The Mathematics", eq. M_states(p, N_d): bytes per parameter of
    // the replicated classes times psi, plus the sharded classes times S.
    static const uint64_t replicated[4] = {16, 4, 2, 0};
    static const uint64_t sharded[4] = {0, 12, 14, 16};
    uint64_t a, b, total;
    if (!mul_ok(replicated[stage], psi, &a) || !mul_ok(sharded[stage], lay.shard_len, &b) ||
        !add_ok(a, b, &total))
        return ZERO_EOVERFLOW;
    *out_bytes = total;
    return ZERO_OK;
}

extern "C" int zero_comm_volume(uint32_t stage, uint64_t psi, uint32_t nd, uint32_t align,
                                zero_comm *out) {
    if (!out || stage > 3)
        return ZERO_EINVAL;
    zero_layout lay;
    int rc = zero_shard_layout(psi, nd, 0, align, &lay);
    if (rc != ZERO_OK)
        return rc;
    // [16B] "The part that sounds too good: communication": a reduce-scatter
    // and an all-gather per step (stages 0-2), one more all-gather of the
    // parameters in stage 3; each ring pass sends nd - 1 shards per rank.
    const uint64_t passes = stage == 3 ? 3 : 2;
    uint64_t volume, per_pass, ring;
    if (!mul_ok(passes, psi, &volume) || !mul_ok((uint64_t)(nd - 1), lay.shard_len, &per_pass) ||
        !mul_ok(passes, per_pass, &ring))
        return ZERO_EOVERFLOW;
    out->passes = passes;
    out->volume_elems = volume;
    out->ring_send_elems = ring;
    return ZERO_OK;
}

extern "C" int zero_adam_scalars(const zero_adam_hparams *hp, uint64_t t, float out[8]) {
    if (!hp || !out || t == 0)
        return ZERO_EINVAL;
    const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps;
    if (!isfinite(lr) || !isfinite(eps) || eps < 0.0 || hp->weight_decay != 0.0)
        return ZERO_EINVAL;
    if (!(b1 >= 0.0 && b1 < 1.0) || !(b2 >= 0.0 && b2 < 1.0))
        return ZERO_EINVAL;
    // Each constant is formed in double and rounded to fp32 once.
    const double td = (double)t;
    out[0] = (float)lr;
    out[1] = (float)b1;
    out[2] = (float)(1.0 - b1);
    out[3] = (float)b2;
    out[4] = (float)(1.0 - b2);
    out[5] = (float)(1.0 - pow(b1, td));
    out[6] = (float)(1.0 - pow(b2, td));
    out[7] = (float)eps;
    return ZERO_OK;
}

extern "C" const char *zero_status_str(int status) {
    switch (status) {
    case ZERO_OK: return "ok";
    case ZERO_EINVAL: return "invalid argument";
    case ZERO_EOVERFLOW: return "size overflows 64 bits";
    case ZERO_EHIP: return "HIP runtime or launch error";
    case ZERO_ENOMEM: return "allocation failed";
    case ZERO_ENOTSUP: return "host CPU lacks AVX2 and F16C";
    case ZERO_ERANGE: return "beyond the fixed limits of the allocation-free step";
    default: return "unknown status";
    }
}

namespace zs {

void pick_vector_path(const uintptr_t *f16, int n16, const uintptr_t *f32, int n32,
                      uint32_t max_width, uint32_t *vec, uint32_t *head) {
    for (uint32_t w : {8u, 4u}) {
        if (w > max_width)
            continue;
        const uintptr_t a16 = 2u * w; // bytes one fp16 vector spans
        for (uint32_t h = 0; h < w; h++) {
            bool ok = true;
            for (int i = 0; i < n16 && ok; i++)
                ok = (f16[i] + 2u * h) % a16 == 0;
            for (int i = 0; i < n32 && ok; i++)
                ok = (f32[i] + 4u * h) % 16u == 0;
            if (ok) {
                *vec = w;
                *head = h;
                return;
            }
        }
    }
    *vec = 1;
    *head = 0;
}

void adam_access_path(uintptr_t p, uintptr_t g, const uintptr_t a32[3], uint64_t n,
                      TensorDesc *d) {
    const uintptr_t a16[2] = {p, g};
    d->pshift = 0;
    d->gshift = 0;
    pick_vector_path(a16, 2, a32, 3, 4, &d->vec, &d->head);
    if (d->vec != 4 && n >= kTileAlignMinElems) {
        // a 16-bit array out of phase: the fp32 arrays by vectors at their
        // head, the parameter's stores and the gradient's loads shifted by
        // their own phase there (one of the two is then not 0)
        pick_vector_path(nullptr, 0, a32, 3, 4, &d->vec, &d->head);
        if (d->vec == 4) {
            d->pshift = (uint32_t)((p / 2u + d->head) % 4u);
            d->gshift = (uint32_t)((g / 2u + d->head) % 4u);
        }
    }
    if (d->vec == 4)
        d->head = adam_head_of(a32, d->head, n);
}

uint32_t adam_head_of(const uintptr_t a32[3], uint32_t vec_head, uint64_t n) {
    if (n < kTileAlignMinElems)
        return vec_head;
    uint32_t ph[3];
    for (int i = 0; i < 3; i++)
        ph[i] = (uint32_t)(((kTileAlignBytes - a32[i] % kTileAlignBytes) % kTileAlignBytes) / 4u);
    if (ph[0] != ph[1] || ph[1] != ph[2] || ph[0] % 4u != vec_head)
        return vec_head;
    return ph[0];
}

bool writes_overlap(Range *r, size_t n) {
    std::sort(r, r + n, [](const Range &a, const Range &b) { return a.lo < b.lo; });
    // Sweep keeping the furthest end seen among written and among all ranges.
    uintptr_t end_any = 0, end_written = 0;
    for (size_t i = 0; i < n; i++) {
        const Range &x = r[i];
        if (x.lo < end_written)
            return true;
        if (x.written && x.lo < end_any)
            return true;
        end_any = std::max(end_any, x.hi);
        if (x.written)
            end_written = std::max(end_written, x.hi);
    }
    return false;
}

bool writes_overlap(std::vector<Range> &r) { return writes_overlap(r.data(), r.size()); }

// The chunk a plan gets when the caller leaves it to the library: the
// largest of kDefaultChunk, kDefaultChunk / 2, ..., kTile whose workgroup
// slots (chunks times kTile-element tiles per chunk) exceed the tiles that
// hold work by at most one eighth.  Big tensors keep
// the compact table of kDefaultChunk; many small tensors get small chunks,
// so that few workgroups start only to find their tile past the end of a
// short chunk.
uint32_t pick_chunk(const TensorDesc *tensors, size_t n) {
    for (uint32_t C = kDefaultChunk; C > kTile; C /= 2) {
        uint64_t slots = 0, work = 0;
        for (size_t k = 0; k < n; k++) {
            const TensorDesc &d = tensors[k];
            const uint64_t body = d.n - std::min<uint64_t>(d.head, d.n);
            const uint64_t chunks = body == 0 ? 1 : (body + C - 1) / C;
            slots += chunks * (C / kTile);
            work += body == 0 ? 1 : (body + kTile - 1) / kTile;
        }
        if (slots <= work + work / 8)
            return C;
    }
    return kTile;
}

int describe_tensor(const zero_tensor &t, TensorDesc *d, Range r[5]) {
    const uintptr_t p = (uintptr_t)t.param_f16, g = (uintptr_t)t.grad_f16,
                    w = (uintptr_t)t.master, m = (uintptr_t)t.m, v = (uintptr_t)t.v;
    if (!p || !g || !w || !m || !v)
        return ZERO_EINVAL;
    if ((p | g) % 2 || (w | m | v) % 4)
        return ZERO_EINVAL;
    uint64_t b2, b4;
    if (!mul_ok(t.n, 2, &b2) || !mul_ok(t.n, 4, &b4))
        return ZERO_EOVERFLOW;
    for (uintptr_t a : {p, g})
        if (a + b2 < a)
            return ZERO_EOVERFLOW;
    for (uintptr_t a : {w, m, v})
        if (a + b4 < a)
            return ZERO_EOVERFLOW;
    r[0] = {p, p + b2, true};
    r[1] = {g, g + b2, false};
    r[2] = {w, w + b4, true};
    r[3] = {m, m + b4, true};
    r[4] = {v, v + b4, true};
    memset(d, 0, sizeof(*d));
    d->p = (uint16_t *)t.param_f16;
    d->g = (const uint16_t *)t.grad_f16;
    d->w = t.master;
    d->m = t.m;
    d->v = t.v;
    d->n = t.n;
    const uintptr_t a32[3] = {w, m, v};
    adam_access_path(p, g, a32, t.n, d);
    return ZERO_OK;
}

void plan_stats(const TensorDesc *tensors, size_t n_desc, uint64_t n_tensors, uint64_t C,
                zero_plan_stats *s) {
    memset(s, 0, sizeof(*s));
    s->n_tensors = n_tensors;
    s->chunk_elems = C;
    for (size_t k = 0; k < n_desc; k++) {
        const TensorDesc &d = tensors[k];
        s->n_params += d.n;
        s->n_chunks += chunks_of(d, C);
        if (d.vec == 1) {
            s->scalar_elems += d.n;
        } else {
            // the head's first head % 4 elements go singly and the rest of
            // it by fours; every chunk body but the tensor's last is a whole
            // number of tiles, so only the tensor's last fewer-than-four
            // elements go singly too
            const uint64_t singles = std::min<uint64_t>(d.head % 4u, d.n);
            const uint64_t vec = (d.n - singles) / 4 * 4;
            s->vector_elems += vec;
            s->scalar_elems += d.n - vec;
        }
    }
    // at most 1/8 of the elements single and the default chunk: the fine
    // tile.  scalar_elems * 8 cannot wrap: the three fp32 arrays of every
    // tensor are disjoint ranges of the address space, so n_params < 2^64 / 12.
    s->tile_elems =
        s->scalar_elems * 8 <= s->n_params && C == kDefaultChunk ? kAdamTileFine : kTile;
    s->table_bytes = n_desc * sizeof(TensorDesc) + s->n_chunks * sizeof(Chunk);
    if (s->tile_elems == kAdamTileFine) {
        s->wg_per_cu = adam_per_cu(kAdamTileFine);
        return;
    }
    // coarse tile: count the tiles that hold elements and those that do
    // more than stream one full tile (a head, a tensor's partial last tile)
    uint64_t work = 0, irregular = 0;
    for (size_t k = 0; k < n_desc; k++) {
        const TensorDesc &d = tensors[k];
        const uint64_t h = d.vec == 4 ? std::min<uint64_t>(d.head, d.n) : 0, body = d.n - h;
        const uint64_t t = body == 0 ? 1 : (body + kTile - 1) / kTile;
        const uint64_t odd = (h > 0 ? 1u : 0u) + (body % kTile != 0 ? 1u : 0u);
        work += t;
        irregular += t == 1 ? std::min<uint64_t>(odd, 1) : odd;
    }
    s->wg_per_cu = adam_per_cu_coarse(work, irregular, s->n_params);
}

int build_host_plan(const zero_tensor *tensors, uint32_t n_tensors, uint32_t chunk_elems,
                    HostPlan *out) {
    if (!out || (n_tensors > 0 && !tensors))
        return ZERO_EINVAL;
    const bool automatic = chunk_elems == 0;
    if (!automatic &&
        (chunk_elems % kTile != 0 || chunk_elems < kMinChunk || chunk_elems > kMaxChunk))
        return ZERO_EINVAL;
    HostPlan plan;
    std::vector<Range> ranges;
    uint64_t n_params = 0;
    for (uint32_t k = 0; k < n_tensors; k++) {
        const zero_tensor &t = tensors[k];
        if (t.n == 0)
            continue;
        TensorDesc d;
        Range r[5];
        const int rc = describe_tensor(t, &d, r);
        if (rc != ZERO_OK)
            return rc;
        ranges.insert(ranges.end(), r, r + 5);
        if (!add_ok(n_params, t.n, &n_params))
            return ZERO_EOVERFLOW;
        plan.tensors.push_back(d);
    }
    if (writes_overlap(ranges))
        return ZERO_EINVAL;

    const uint64_t C =
        automatic ? pick_chunk(plan.tensors.data(), plan.tensors.size()) : chunk_elems;
    for (uint32_t k = 0; k < (uint32_t)plan.tensors.size(); k++) {
        const TensorDesc &d = plan.tensors[k];
        const uint64_t nc = chunks_of(d, C);
        for (uint64_t j = 0; j < nc; j++)
            plan.chunks.push_back(chunk_of(d, k, C, j));
    }
    plan_stats(plan.tensors.data(), plan.tensors.size(), n_tensors, C, &plan.stats);
    *out = std::move(plan);
    return ZERO_OK;
}

} // namespace zs

extern "C" int zero_plan_describe(const zero_tensor *tensors, uint32_t n_tensors,
                                  uint32_t chunk_elems, zero_plan_stats *out) {
    if (!out)
        return ZERO_EINVAL;
    zs::HostPlan plan;
    int rc = zs::build_host_plan(tensors, n_tensors, chunk_elems, &plan);
    if (rc == ZERO_OK)
        *out = plan.stats;
    return rc;
}
