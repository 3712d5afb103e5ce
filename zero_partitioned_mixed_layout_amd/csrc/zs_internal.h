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
    uint32_t vec;      // 4: four-element vector path; 1: single elements
    uint32_t head;     // leading elements peeled before the first tile (vector
                       // path: head % 4 singly, then by fours; see adam_head_of)
    uint32_t pshift;   // vector path: the parameter's element phase mod 4 at
                       // the vector-aligned elements (0: its stores are 8-byte
                       // vectors too; 1-3: shifted, see adam_access_path)
    uint32_t gshift;   // the same for the gradient (1-3: shifted loads)
};
static_assert(sizeof(TensorDesc) == 64, "TensorDesc is 64 bytes");

// One work item of a workgroup: `count` elements of tensor `tensor` from
// element `start` (16 bytes).  Chunk starts other than a tensor's first are
// vector-aligned, and every chunk but a tensor's last holds a whole number
// of wave tiles (plus the peeled head in a tensor's first chunk).
struct Chunk {
    uint32_t tensor;
    uint32_t count;
    uint64_t start;
};
static_assert(sizeof(Chunk) == 16, "Chunk is 16 bytes");

// Lanes of a wave, and threads of every workgroup of both kernels: one wave
// per workgroup.
constexpr uint32_t kWave = 64;

// Elements of one wave tile of the reduce and fused kernels (64 lanes x two
// groups of four), and the unit of a plan's chunk sizes.
constexpr uint32_t kTile = 512;

// Elements of an Adam wave tile, chosen per plan: kAdamTileFine (64 lanes x
// one group of four) when at least 7/8 of the plan's elements take the
// vector path and its chunk is kDefaultChunk (big tensors), else kTile (two
// groups of four per lane).  Measured on MI355X, each against the other in
// one process: the fine tile is 1-5% faster on flat shards of 117M-937.5M
// elements (1.4% slower on one of 102.4M), 0.6-2% on the Llama-7B and
// GPT-2-XL lists in flattened buffers
// and 7-10% on the same lists held as five allocations per tensor; the
// coarse tile is 4-7% faster on the single-element path (a lane keeps
// twice the loads in flight) and 4% on 100,000 tensors of 1,024 elements.
constexpr uint32_t kAdamTileFine = 256;
static_assert(kTile % kAdamTileFine == 0, "chunks hold whole Adam tiles");

// Chunk sizes a plan accepts (multiples of kTile) and the default.  One
// workgroup updates one Adam tile; the chunk size only sets how many tiles
// share a table entry (a tensor's short last chunk leaves some workgroups
// idle).
constexpr uint32_t kMinChunk = kTile;
constexpr uint32_t kMaxChunk = 1u << 24;
constexpr uint32_t kDefaultChunk = 16384;

// Largest grid of every kernel, in one-wave workgroups: the most whose
// work-items (64 each) still fit the 32-bit grid size of a dispatch.  Larger
// work strides over it.  Measured on MI355X with the Llama-7B list (26.3M
// Adam tiles): a grid capped at 2^24 that strode over the rest ran 2-3%
// slower than one workgroup per tile.
constexpr uint64_t kMaxGrid = (1ull << 26) - 1;
static_assert(kMaxGrid * kWave <= 0xFFFFFFFFull, "grid size fits 32 bits");

// Resident one-wave workgroups per CU for the Adam step, by tile: each
// keeps four (fine) or eight (coarse) 8- or 16-byte loads per lane in
// flight.  Measured on MI355X: the fine tile is fastest at 12 (over 10..14)
// on flat shards of 117M-3G elements and on both lists in either layout;
// the coarse tile at 7 (over 5..8) on flat shards of 117M-6.7G elements.
inline uint32_t adam_per_cu(uint32_t tile) { return tile == kAdamTileFine ? 12u : 7u; }

// The coarse tile's cap for a plan whose `work` tiles hold elements, of
// which `irregular` hold a tensor's head or its partial last tile.  Such
// tiles carry fewer bytes and a partial one also more loads per lane, so a
// plan of many of them needs more waves in flight: with fewer than one
// irregular tile in 200 the cap stays at 7, else it is 7 * 512 / e + 7
// within 14..27 (19 and 21 taken as 20 and 22, the counts their LDS
// reservation admits), where e is the average element count of a tile with
// work.  Measured on MI355X (lists in flattened buffers at their packed
// offsets, caps 7..28 and uncapped, one process each; fraction of 8 TB/s
// at the best cap against cap 7): 100,000 x 1,024 (no irregular tiles)
// best at 7; 20,000 of 1-8,000 elements 0.655 at 14-18 against 0.608;
// 50,000 of 1-2,000 0.673 at 14 against 0.531; 100,000 of 1-600 0.542 at
// 18-22 against 0.325; 100,000 x 300 0.510 at 14 against 0.376; 100,000 x
// 100 0.461 uncapped (28, as many as the kernel's registers allow) against
// 0.229.  With partial tiles updated in one pass (adam_span_g), caps 7-24
// in one process: one tensor of 117M and the GPT-2-XL list on 512-element
// tiles (0.04% irregular tiles) best at 7-8; 1,000 tensors of 1-100,000
// (2%) 0.714-0.717 at 10-12 and 0.709 at 14 against 0.690 at 7, hence the
// threshold of one in 200 (it was one in 20).
inline uint32_t adam_per_cu_coarse(uint64_t work, uint64_t irregular, uint64_t n_params) {
    if (work == 0 || irregular * 200 < work)
        return 7u;
    const double e = (double)n_params / (double)work;
    const double k = 7.0 * kTile / (e > 1.0 ? e : 1.0) + 7.0;
    const uint32_t r = k < 14.0 ? 14u : (k > 27.0 ? 27u : (uint32_t)(k + 0.5));
    // on a 160 KiB CU the LDS reservation for 19 or 21 also admits one
    // more workgroup (no multiple of 256 bytes separates the two): say so
    return r == 19u || r == 21u ? r + 1u : r;
}

// Elements one wave of the parameter gather moves per tile: four 16-byte
// loads per lane in flight on the widest path.
constexpr uint32_t kGatherTile = 2048;

// Resident one-wave workgroups per CU for the parameter gather.  Measured on
// MI355X with 64 shards of 117,187,500 elements: 16 is 1-5% ahead of 8 and
// 12; 1024-element tiles at 16 or 24 and 4096 at 8 were no faster, and
// 512-element tiles without a cap (one vector per lane) 7-12% slower.
constexpr uint32_t kGatherPerCU = 16;

// Bytes of a cache line (the unit of the gather's destination alignment).
constexpr uint32_t kLine = 128;

// Bytes of fp32 that one 256-element Adam tile spans, and the boundary its
// tiles start on where a tensor's fp32 arrays allow it (adam_head_of).
constexpr uint32_t kTileAlignBytes = 4u * kAdamTileFine;

// Smallest tensor whose head runs to that boundary.  Tile 0 finishes the
// head before it loads its own elements, one more pass over memory, which
// costs more than the alignment saves on small tensors.  Measured on MI355X,
// lists at random offsets in flattened buffers, head to 1 KiB against the
// vector head alone, one process: sizes 1-1,024 elements 0.410 against
// 0.423 of 8 TB/s; 1,024-4,096 0.571 against 0.558; 4,096-16,384 0.613
// against 0.562; 16,384-65,536 0.647 against 0.597.
constexpr uint64_t kTileAlignMinElems = 1024;

// Elements per chunk of the offload pipeline (8 MiB of fp16 per staging
// buffer).
constexpr uint64_t kOffloadChunk = 4ull << 20;

// Slices whose fp16 vectors one lane keeps in flight at once when reducing
// nd slices in batches of 16, 8, 4, then 1 (the fused kernel and the
// reduce's 8-byte and single-element paths).
inline uint32_t slices_in_flight(uint32_t nd) {
    return nd >= 16 ? 16 : (nd >= 8 ? 8 : (nd >= 4 ? 4 : 1));
}

// Resident one-wave workgroups per CU for the reduction over nd slices in
// batches of 16, 8, 4 and 1 (the 16-byte path before it took the rest
// after the batches of 16 in one batch; the other paths derive their caps
// from this): about 64 16-byte vectors per lane in flight per CU, at most 16
// workgroups (16 with 1-7 slices, 8 with 8-15), and with 16 slices in
// flight 4, raised to 5 and 6 when a lane runs only two or one batch of 16
// (a shorter-lived wave needs more of them).  Measured on MI355X over
// 117,187,500 elements, one process per sweep of caps 3-32, fraction of
// 8 TB/s at the chosen cap against the former one: N_d = 1 0.532 (16)
// against 0.310 (8); 2 0.561 against 0.318; 3 0.579 against 0.329; 4 0.881
// against 0.662; 5 0.866 against 0.587; 6 0.835 against 0.538; 7 0.803
// against 0.506; 8 and 12 best at 8 (0.853, 0.831); 16 0.836 (6) against
// 0.767 (4); 24 0.825 (5) against 0.786; 32 0.827 (5) against 0.816; 48
// and 64 best at 4 (0.839, 0.837).
inline uint32_t reduce_per_cu(uint32_t nd) {
    const uint32_t sif = slices_in_flight(nd);
    if (sif < 16) {
        const uint32_t k = (64 + sif - 1) / sif;
        return k > 16 ? 16 : k;
    }
    const uint32_t batches = (nd + 15) / 16;
    return batches == 1 ? 6 : (batches == 2 ? 5 : 4);
}

// The same for the reduce's 16-byte path (zs_reduce_kernel, one group of
// eight per lane), which loads batches of 16 slices and then the rest in
// one batch, every load of a batch in flight before its first add.
// Measured on MI355X over 117,187,500 elements, caps 4-16 in one process
// (fraction of 8 TB/s at 2 N_d + 2 bytes per element, best cap, against
// batches of 16, 8, 4 and 1 at their caps): N_d = 5 0.880 at 12 (0.846),
// 6 0.863 at 10 (0.813), 7 0.843 at 10 (0.785), 9-11 0.820-0.840 at 8
// (0.656-0.758), 13 0.808 at 8 (0.770), 14-15 0.817-0.821 at 6
// (0.694-0.726), 17 0.812 at 8 (0.734), 19-23 0.804-0.813 at 6
// (0.626-0.784), 28 0.814 at 5 (0.807), 31 0.796 at 5 (0.701); at 4, 8,
// 12, 16, 24, 32 and 64 (the same batches as before, or 12 at once
// against 8 then 4) within 1.1% of the former code.
inline uint32_t reduce_per_cu_vec8(uint32_t nd) {
    if (nd <= 4)
        return 16;
    if (nd == 5)
        return 12;
    if (nd <= 7)
        return 10;
    if (nd <= 13)
        return 8;
    if (nd <= 16)
        return 6;
    if (nd == 17)
        return 8;
    if (nd <= 23)
        return 6;
    return nd <= 32 ? 5 : 4;
}

// Tiles per run of one XCD on the reduce's 8-byte path (zs_reduce_vec4_kernel;
// 0: tiles in launch order).  Its slices sit 8 bytes off their 128-byte
// lines, so neighbouring tiles share a line of each; in launch order they run
// on different XCDs and each XCD's L2 reads it (1.117 times the algorithmic
// bytes from HBM over 64 slices of 117,187,500 elements back to back in one
// buffer).  Measured on MI355X there, one process, runs of 2-12 tiles
// (fraction of 8 TB/s against launch order): runs of 4 at N_d = 8 0.800
// (0.761), 12 0.809 (0.747), 16 0.798 (0.737), 24 0.783 (0.734), 32 0.774
// (0.732), 48 0.756 (0.725), 64 0.757 (0.733); 4 equal (0.828 against
// 0.824); 2 lower at every run (0.644-0.659 against 0.686); runs of 3, 6
// and 12 below those of 2, 4 and 8.  One run per XCD (8 far-apart streams
// per slice) cut the reads to 1.040 times but ran 5% slower at N_d = 64;
// on 16-byte-aligned slices, where no line is shared, runs of 2-8 lost up
// to 9%.
inline uint32_t reduce_vec4_run(uint32_t nd) { return nd >= 4 ? 4u : 0u; }

// The same for the reduce's other access paths.  vec = 4 (slices sharing
// only an 8-byte phase; two 8-byte groups per lane per slice, the same
// batches as the 16-byte path): 24 at 1-2 slices, 12 at 8 (0.754-0.760
// at 10-12 against 0.751 at 8), else the 16-byte path's.
// Measured on MI355X, 117,187,500 elements, slices back to back in one
// buffer (every other one 8 bytes off), caps 4-24 in one process (fraction
// of 8 TB/s, best cap, against batches of 8, 4 and 1 at their former
// caps): N_d = 7 0.772 at 10 (0.739), 12 0.749 at 8 (0.738), 16 0.738 at 6
// (0.718), 17 0.730 at 8 (0.644), 24 0.731 at 6 (0.717), 32 0.724 at 5
// (0.714), 64 0.732 at 4 (0.713); 2, 4 and 8 equal; the table's cap within
// 1.2% of the best at every N_d measured (with batches of 8, 4 and 1 the
// path had 24 with one slice in flight, 0.685 against 0.602 at 16 for
// N_d = 2, and 12 with eight).  vec = 1 (no common phase; eight single
// elements per lane per slice, batches of 8 slices and then the rest in
// one, half the bytes): 24 at 1-2 slices, 16 at 3, 12 at 4-5, 8 at 6-23, 6
// from 24.  Measured on MI355X, 117,187,501 elements, slices back to back
// in one buffer (every 2-byte phase), caps 4-24 in one process (fraction
// of 8 TB/s against batches of 8, 4 and 1 at twice reduce_per_cu's cap, at
// most 24, 8 with eight slices in flight): N_d = 2 0.724 at 24 (0.664), 3
// 0.728 at 16 (0.691), 4-5 0.706-0.712 at 12 (0.672-0.680), 6-7
// 0.687-0.707 at 8 (0.655-0.659), 8 0.697 (0.698), 11-16 0.681-0.691 at 8
// (0.623-0.659), 24-64 0.662-0.668 at 6 (0.651-0.660).
inline uint32_t reduce_per_cu_path(uint32_t nd, uint32_t vec) {
    if (vec == 4)
        return nd <= 2 ? 24u : (nd == 8 ? 12u : reduce_per_cu_vec8(nd));
    if (vec == 1)
        return nd <= 2 ? 24u : (nd == 3 ? 16u : (nd <= 5 ? 12u : (nd < 24 ? 8u : 6u)));
    return reduce_per_cu_vec8(nd);
}

// The same for zs_reduce_few_kernel (1-3 slices, four groups per lane, 4 N_d
// 16-byte loads per lane in flight): about 100 such loads per lane per CU.
// Measured on MI355X over 117,187,500 elements, caps 8-28 in one process
// (fraction of 8 TB/s at 2 N_d + 2 bytes per element, against 0.521 /
// 0.554 / 0.577 with one group per lane): N_d = 1 0.861-0.868 at 24-28
// (0.845 at 16), N_d = 2 0.867-0.868 at 16-20, N_d = 3 0.853 at 8 (0.844 at
// 12, 0.828 at 16).
// With eight groups of four per lane (vec = 4, slices that share only an
// 8-byte phase, the same 32 elements per lane), over 117,187,500 elements,
// caps 8-28 in one process, against one 512-element tile per wave with
// batches of one slice: N_d = 1 0.854 at 28 (0.495), 2 0.854 at 16 (0.680),
// 3 0.848 at 12 (0.801).
inline uint32_t reduce_per_cu_few(uint32_t nd, uint32_t vec) {
    if (vec == 4)
        return nd == 1 ? 28u : (nd == 2 ? 16u : 12u);
    return nd == 1 ? 27u : (nd == 2 ? 16u : 8u);
}

// Whether the fused step's 16-byte path loads a tile's fp32 state after the
// slices (then it arrives while the reduced gradients cross the LDS) instead
// of with the first slice batch.  Measured on MI355X, one process, 937.5M
// elements: after is 3.6% faster at N_d = 4 and 2.5% at N_d = 8 (with the
// caps below); before is 4-5% faster at N_d = 16 and equal at N_d = 64.
inline bool fused_state_late(uint32_t nd) { return slices_in_flight(nd) < 16; }

// Slices from which zero_reduce_adam_step runs the reduce and then the Adam
// step (two kernels) instead of the fused kernel.  Measured on MI355X,
// 117,187,500 elements, one process per N_d, with the caps of this file,
// fused kernel time over the two kernels': 0.816 at N_d = 1, 0.826 at 2,
// 0.904 at 4, 0.965 at 8, 0.967 at 12; 1.016 at 16, 0.988 at 20, 1.007 at
// 24, 1.034 at 28, 1.124 at 31 (from 16 slices its mix of state writes
// into the slice reads costs about what the 4 bytes per element it saves
// gain).
constexpr uint32_t kFusedSplitSlices = ZERO_FUSED_SPLIT_SLICES;

// Resident one-wave workgroups per CU for the fused reduce + Adam step.
// State first (the 8-byte and single-element paths, and the 16-byte path
// from 16 slices): about 70 16-byte vectors per lane in flight per CU,
// counting the six fp32 state vectors issued with the first slice batch (4
// workgroups at N_d >= 16, 5 at N_d = 8: the measured optima), between 2
// and 8.  State last (the 16-byte path below 16 slices, which loads all of
// its 1-15 slices as one batch): 12 at one slice, 8 at 2-6, 6 at 7-10 and
// 5 at 11-15.  Measured on MI355X over 117,187,500 elements, caps 4-20, one
// process (fraction of 8 TB/s at 2 N_d + 26 bytes per element, against the
// former batches of 8, 4 and 1 at their caps): N_d = 1 0.792 at 12 (0.789),
// 2 0.783 at 8 (0.785), 3 0.795 at 8 (0.772), 5 0.804 at 8 (0.782), 6
// 0.753-0.781 at 8 (0.741-0.747), 7 0.772 at 6 (0.707), 9-10 0.784-0.788
// at 6 (0.711-0.755), 11 0.761-0.763 at 5 (0.670-0.671), 13-15 0.772-0.778
// at 5 (0.690-0.765); 4, 8 and 12 within 0.4% of the former code.
// The 8-byte path (vec = 4, state first, its 1-15 slices below 16 as one
// batch) takes about 75 vectors with all of those slices counted: 8 at 1-4
// slices, 7 at 5-6, 6 at 7-8, 5 at 9-12, 4 from 13.  Measured
// over 117,187,500 elements, slices back to back in one buffer (every other
// one 8 bytes off), caps 3-10 in one process (fraction of 8 TB/s against
// batches of 8, 4 and 1 at the former caps): N_d = 2 0.783 at 8 (0.757), 3
// 0.769 at 8 (0.714), 5 0.743 at 8 (0.721), 7 0.747 at 6 (0.654), 9 0.759
// at 6 (0.728), 11 0.751 at 5 (0.647), 15 0.726 at 4 (0.639); 4, 8 and 12
// equal; the rule within 1% of the best cap at every N_d measured.
// The single-element path (vec = 1, no common phase; batches of 8 slices
// and then the rest in one, half the bytes per wave) takes 8 at 1-5 slices
// and 6 from 6: over 117,187,501 elements, slices back to back in one
// buffer (every 2-byte phase), caps 4-16 in one process, against twice the
// state-first rule above (10-16): N_d = 2 0.726 (0.704), 3 0.707 (0.685), 5
// 0.694 (0.677), 7 0.673 (0.662), 8 0.685 (0.663), 11 0.695 (0.666), 15
// 0.671 (0.650); a second process: 2 0.709 (0.716), 8 0.720 (0.719), 11
// 0.690 (0.667).
inline uint32_t fused_per_cu(uint32_t nd, bool state_late, uint32_t vec = 8) {
    const uint32_t sif = slices_in_flight(nd);
    if (vec == 1)
        return nd <= 5 ? 8u : 6u;
    if (state_late)
        return nd == 1 ? 12u : (nd <= 6 ? 8u : (nd <= 10 ? 6u : 5u));
    const uint32_t in_flight = vec == 4 ? (nd < 16 ? nd : 16u) : sif;
    const uint32_t target = vec == 4 ? 75u : 70u;
    const uint32_t per_wave = 6 + in_flight;
    const uint32_t k = (target + per_wave - 1) / per_wave;
    return k < 2 ? 2 : (k > 8 ? 8 : k);
}

// A tensor's chunks: the first holds its peeled head plus up to C
// elements, every later one C elements (the tensor's last may be shorter).
// constexpr, so that the device code that fills a table on the GPU uses the
// same formulas as the host plan builder (HIP compiles constexpr functions
// for both sides).
constexpr uint64_t first_chunk_count(const TensorDesc &d, uint64_t C) {
    const uint64_t head = d.head < d.n ? d.head : d.n;
    return d.n < head + C ? d.n : head + C;
}
constexpr uint64_t chunks_of(const TensorDesc &d, uint64_t C) {
    const uint64_t first = first_chunk_count(d, C);
    return 1 + (d.n - first + C - 1) / C;
}
// Chunk j of tensor k (j < chunks_of(d, C)).
constexpr Chunk chunk_of(const TensorDesc &d, uint32_t k, uint64_t C, uint64_t j) {
    const uint64_t first = first_chunk_count(d, C);
    if (j == 0)
        return {k, (uint32_t)first, 0};
    const uint64_t start = first + (j - 1) * C;
    const uint64_t left = d.n - start;
    return {k, (uint32_t)(left < C ? left : C), start};
}

struct HostPlan {
    std::vector<TensorDesc> tensors;
    std::vector<Chunk> chunks;
    zero_plan_stats stats;
};

// A byte range [lo, hi) of one array, and whether the call writes it.
struct Range {
    uintptr_t lo, hi;
    bool written;
};

// Validate and classify; fills `out`.  chunk_elems: 0 for the library's
// choice (kDefaultChunk unless the tensors are small: see pick_chunk), else
// a multiple of kTile in [kMinChunk, kMaxChunk].  Pure host code.
int build_host_plan(const zero_tensor *tensors, uint32_t n_tensors, uint32_t chunk_elems,
                    HostPlan *out);

// The Adam step's peeled head of a tensor of n elements on the
// four-element vector path, given its vector head (the fewer than four
// elements before the first vector) and its fp32 master, m and v
// addresses.  When n >= kTileAlignMinElems and the three reach a 1 KiB
// boundary at the same element, the head runs up to that element (fewer
// than 256, equal to the vector head mod 4), so that every full tile after
// it starts on 1 KiB of fp32; otherwise it is the vector head.  The fp32
// arrays carry 24 of the step's 28 bytes per parameter.  Measured on
// MI355X with the GPT-2-XL list packed in flattened buffers (its 1,600-
// element tensors put the big ones at multiples of 64 elements): tiles at
// the tensors' own offsets ran at 0.788 of 8 TB/s, tiles on 1 KiB at
// 0.812-0.816, as fast as one flat tensor of the same size.
uint32_t adam_head_of(const uintptr_t a32[3], uint32_t vec_head, uint64_t n);

// The Adam step's access path for a tensor of n elements (its parameter p,
// gradient g and fp32 master, m, v at a32): sets d->vec, d->head, d->pshift
// and d->gshift.  The vector path when all five arrays agree in phase after
// peeling at most 3 elements (both shifts 0); else, on a tensor of
// kTileAlignMinElems or more whose fp32 arrays agree, the vector path with
// the parameter stored shifted (pshift 1-3: its element phase mod 4 at the
// vector-aligned elements) and the gradient loaded shifted (gshift 1-3)
// where either is out of phase; otherwise single elements (vec 1).  A ZeRO
// rank's 16-bit arrays are often views of full buffers at an offset that
// is not a multiple of four elements.  Measured on MI355X, plans over the
// same buffers in one process (fraction of 8 TB/s, shifted against
// single): the parameter 1-3 elements off, one tensor of 117,187,500
// elements 0.747-0.764 against 0.682-0.692, the GPT-2-XL list 0.738-0.751
// against 0.560-0.570, random sizes 1-8,192 0.637 against 0.607 and
// 1-100,000 0.660 against 0.643; the gradient off too, 0.739-0.745 against
// 0.681-0.682 (117M) and 0.731-0.734 against 0.629-0.631 (GPT-2-XL); the
// gradient alone off, 0.774-0.788 against 0.707-0.708.  Below 1,024
// elements single elements were faster (random sizes 1-1,024: 0.616 with
// the rule against 0.551 shifted).
void adam_access_path(uintptr_t p, uintptr_t g, const uintptr_t a32[3], uint64_t n,
                      TensorDesc *d);

// Whether any of the descriptors is on the vector path with a 16-bit array
// out of phase: the Adam kernels are built twice, with the shifted modes
// and without them (so that in-phase plans run the in-phase tile code
// alone: measured 0.3% faster than with the modes compiled in).
inline bool any_shift(const TensorDesc *d, size_t n) {
    for (size_t k = 0; k < n; k++)
        if (d[k].vec == 4 && (d[k].pshift | d[k].gshift) != 0)
            return true;
    return false;
}

// One non-empty tensor: its descriptor (vector path and peeled head) and the
// byte ranges of its five arrays (param, grad, master, m, v).  Errors:
// EINVAL (a NULL or misaligned array), EOVERFLOW.
int describe_tensor(const zero_tensor &t, TensorDesc *d, Range r[5]);

// The library's chunk for these descriptors (see build_host_plan).
uint32_t pick_chunk(const TensorDesc *tensors, size_t n);

// Plan statistics of these descriptors cut into chunks of C elements;
// n_tensors counts the caller's tensors, empty ones included.
void plan_stats(const TensorDesc *tensors, size_t n_desc, uint64_t n_tensors, uint64_t C,
                zero_plan_stats *s);

// True if two of the ranges overlap where at least one of them is written
// (read-only ranges may overlap each other).  Sorts r.
bool writes_overlap(Range *r, size_t n);
bool writes_overlap(std::vector<Range> &r);

// Pick the widest vector width, at most max_width (8 or 4; else 1), and the
// leading-element peel (< width) for which every address is aligned: fp16
// arrays need 2*width bytes, fp32 arrays 16 bytes.
void pick_vector_path(const uintptr_t *f16, int n16, const uintptr_t *f32, int n32,
                      uint32_t max_width, uint32_t *vec, uint32_t *head);

} // namespace zs

#endif
