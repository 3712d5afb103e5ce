// Host code of the library (layout, ledgers, plan classification, step
// scalars, the host Adam step) driven over ragged and invalid inputs; built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// test_host_sanitize.py.  No device calls.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#include <vector>
#include <random>
#include "zero_shard.h"

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { printf("FAIL %s at %d\n", #c, __LINE__); fails++; } } while (0)

int main() {
    // layout + ledger + comm over a brute-force range
    for (uint64_t psi = 0; psi < 300; psi += 7)
        for (uint32_t nd = 1; nd < 10; nd++)
            for (uint32_t al : {1u, 2u, 3u, 8u, 512u})
                for (uint32_t r = 0; r < nd; r++) {
                    zero_layout L;
                    EXPECT(zero_shard_layout(psi, nd, r, al, &L) == 0);
                    for (uint32_t st = 0; st < 4; st++) {
                        uint64_t b; EXPECT(zero_state_bytes(st, psi, nd, al, &b) == 0);
                        zero_comm c; EXPECT(zero_comm_volume(st, psi, nd, al, &c) == 0);
                    }
                }
    zero_layout L;
    EXPECT(zero_shard_layout(UINT64_MAX, 3, 0, 512, &L) != 0);
    EXPECT(zero_shard_layout(10, 0, 0, 1, &L) != 0);
    EXPECT(zero_shard_layout(10, 2, 2, 1, &L) != 0);
    uint64_t b;
    EXPECT(zero_state_bytes(0, UINT64_MAX / 8, 1, 1, &b) != 0);
    EXPECT(zero_state_bytes(4, 10, 1, 1, &b) != 0);
    // plan describe over ragged lists with every alignment class
    std::mt19937_64 rng(1);
    for (int trial = 0; trial < 300; trial++) {
        int nt = 1 + rng() % 40;
        std::vector<zero_tensor> ts(nt);
        uintptr_t base = (uintptr_t)1 << 40;
        for (int k = 0; k < nt; k++) {
            uint64_t n = rng() % 5000;
            if (rng() % 7 == 0) n = rng() % 3;
            auto off = [&](int sz) { uintptr_t a = base + (rng() % 8) * sz; base += (n + 64) * sz + 4096; return a; };
            ts[k].param_f16 = (void *)off(2);
            ts[k].grad_f16 = (const void *)off(2);
            ts[k].master = (float *)off(4);
            ts[k].m = (float *)off(4);
            ts[k].v = (float *)off(4);
            ts[k].n = n;
        }
        zero_plan_stats s;
        uint64_t chunk = (trial % 3 == 0) ? 0 : 512ull * (1 + rng() % 40);
        int rc = zero_plan_describe(ts.data(), nt, chunk, &s);
        EXPECT(rc == 0);
        if (rc == 0) {
            uint64_t tot = 0; for (auto &t : ts) tot += t.n;
            EXPECT(s.n_params == tot && s.vector_elems + s.scalar_elems == tot);
        }
    }
    // invalid plans
    {
        zero_tensor t = {(void *)0x10000, (const void *)0x10000, (float *)0x20000, (float *)0x30000, (float *)0x40000, 100};
        zero_plan_stats s;
        EXPECT(zero_plan_describe(&t, 1, 0, &s) != 0);           // p and g alias
        t.grad_f16 = (const void *)0x50000;
        EXPECT(zero_plan_describe(&t, 1, 0, &s) == 0);
        EXPECT(zero_plan_describe(&t, 1, 511, &s) != 0);         // chunk not a multiple of 512
        EXPECT(zero_plan_describe(&t, 1, (1ull << 24) + 512, &s) != 0);
        EXPECT(zero_plan_describe(nullptr, 1, 0, &s) != 0);
        t.master = (float *)0x20001;                              // misaligned fp32
        EXPECT(zero_plan_describe(&t, 1, 0, &s) != 0);
    }
    // scalars
    zero_adam_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.0};
    float sc[8];
    for (uint64_t t : {1ull, 2ull, 1000ull, 1ull << 40}) EXPECT(zero_adam_scalars(&hp, t, sc) == 0);
    EXPECT(zero_adam_scalars(&hp, 0, sc) != 0);
    // host Adam over ragged sizes and thread counts
    for (uint64_t n : {0ull, 1ull, 3ull, 7ull, 8ull, 9ull, 1000ull, 65537ull, 1000003ull}) {
        for (uint32_t th : {0u, 1u, 3u, 16u}) {
            std::vector<uint16_t> g(n + 1), p(n + 1);
            std::vector<float> w(n + 1), m(n + 1), v(n + 1);
            for (uint64_t i = 0; i < n; i++) { g[i] = (uint16_t)(rng() & 0x3BFF); w[i] = 0.01f * (float)(i % 13); }
            int32_t flag = 0;
            int rc = zero_adam_step_host(g.data(), p.data(), w.data(), m.data(), v.data(), n, &hp, 1, th, &flag);
            EXPECT(rc == 0 || rc == ZERO_ENOTSUP);
            rc = zero_adam_step_host_bf16(g.data(), p.data(), w.data(), m.data(), v.data(), n, &hp, 2, th, &flag);
            EXPECT(rc == 0 || rc == ZERO_ENOTSUP);
        }
    }
    {   // the thread bound: 1025 is rejected, 1024 runs
        std::vector<uint16_t> g(100, 0x3C00), p(100);
        std::vector<float> w(100, 1.f), m(100), v(100);
        EXPECT(zero_adam_step_host(g.data(), p.data(), w.data(), m.data(), v.data(), 100, &hp, 1, 1025, nullptr) == ZERO_EINVAL);
        EXPECT(zero_adam_step_host(g.data(), p.data(), w.data(), m.data(), v.data(), 100, &hp, 1, 1024, nullptr) == 0);
        zero_offload *o = nullptr;
        EXPECT(zero_offload_create(0, 1025, &o) == ZERO_EINVAL && o == nullptr);
    }
    for (int st = -7; st <= 1; st++) EXPECT(zero_status_str(st) != nullptr);
    printf("asan driver: %d failures\n", fails);
    return fails != 0;
}
