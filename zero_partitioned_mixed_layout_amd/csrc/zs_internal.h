// zs_internal.h -- layout of the device chunk table and the host-side plan
// builder shared by the host code and the kernels of libzeroshard.so.
#ifndef ZS_INTERNAL_H
#define ZS_INTERNAL_H

#include <stdint.h>

#include <vector>

#include "zero_shard.h"

namespace zs {

// One tensor of the shard as the kernels see it (64 bytes).
struct TensorDesc {
    uint16_t *p;       // fp16 parameter
    const uint16_t *g; // fp16 gradient
    float *w;          // fp32 master
    float *m;          // fp32 first moment
    float *v;          // fp32 second moment
    uint64_t n;
    uint32_t vec;      // access width in elements: 8, 4 or 1
    uint32_t head;     // leading elements done singly so the rest is aligned
    uint64_t unused;   // pads the descriptor to 64 bytes
};
static_assert(sizeof(TensorDesc) == 64, "TensorDesc is 64 bytes");

// One work item: `count` elements of tensor `tensor` from element `start`
// (16 bytes).  Chunk starts other than a tensor's first are aligned for the
// tensor's vector width.
struct Chunk {
    uint32_t tensor;
    uint32_t count;
    uint64_t start;
};
static_assert(sizeof(Chunk) == 16, "Chunk is 16 bytes");

// Threads per workgroup of both kernels (four 64-wide waves).
constexpr int kBlock = 256;

struct HostPlan {
    std::vector<TensorDesc> tensors;
    std::vector<Chunk> chunks;
    zero_plan_stats stats;
};

// Validate and classify; fills `out`.  Pure host code.
int build_host_plan(const zero_tensor *tensors, uint32_t n_tensors, HostPlan *out);

// Elements per chunk for a plan of n_params elements.
uint64_t chunk_elems_for(uint64_t n_params);

// Pick the widest vector width (8, 4, else 1) and the leading-element peel
// (< width) for which every address is aligned.  fp16 arrays need 2*width
// bytes, fp32 arrays 16 bytes for widths 8 and 4.
void pick_vector_path(const uintptr_t *f16, int n16, const uintptr_t *f32, int n32,
                      uint32_t *vec, uint32_t *head);

} // namespace zs

#endif
