// Drives every C-ABI entry point of rba_host.cpp through valid and invalid
// arguments, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
// (kernel launches are host stand-ins; device pointers are fake addresses
// that are never dereferenced). Exit status 0 = every expectation held.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <thread>
#include <vector>

#include "rba.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "%s:%d: expectation failed: %s (%s)\n", __FILE__, __LINE__, #cond, \
                    rba_last_error());                                      \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static void* P(uintptr_t off = 0) { return reinterpret_cast<void*>(0x100000 + off); }

static rba_attn_params prm(int hq, int hkv, int dv, int R, int W) {
    rba_attn_params p;
    p.num_heads_q = hq;
    p.num_heads_kv = hkv;
    p.head_dim_qk = 128;
    p.head_dim_v = dv;
    p.rel_extent = R;
    p.window = W;
    p.scale = 0.08838834764831845f;
    p.block_size = 128;
    return p;
}

static void prefill_cases() {
    const int Rs[] = {1, 5, 127, 512, 1024};
    const int Hs[][2] = {{32, 8}, {4, 1}, {48, 8}, {12, 2}, {8, 8}, {128, 2}};
    for (int R : Rs)
        for (auto& h : Hs)
            for (int W : {0, 1, 512})
                for (int dv : {64, 128}) {
                    rba_attn_params p = prm(h[0], h[1], dv, R, W);
                    const float* rel = (const float*)P(4);
                    EXPECT(rba_validate_prefill(&p, P(), P(), P(), 64, rel, (const int32_t*)P(), (const int32_t*)P(),
                                                (const int32_t*)P(), 64, 2, 8192, 8192, (const float*)P()) == RBA_OK);
                    EXPECT(rba_prefill(&p, P(), P(), P(), 64, rel, (const int32_t*)P(), (const int32_t*)P(),
                                       (const int32_t*)P(), 64, 2, 8192, 8192, (float*)P(), nullptr, nullptr) == RBA_OK);
                    EXPECT(rba_prefill_gated(&p, P(), P(), P(), 64, rel, (const int32_t*)P(), (const int32_t*)P(),
                                             (const int32_t*)P(), 64, 2, 100, 8192, (const float*)P(4),
                                             (const float*)P(8), (float*)P(), (float*)P(4), nullptr) == RBA_OK);
                    EXPECT(rba_prefill_logpos(&p, P(), P(), P(), 64, rel, (const int32_t*)P(), (const int32_t*)P(),
                                              (const int32_t*)P(), 64, 1, 100, 8192, (const float*)P(4),
                                              (float*)P(), nullptr, nullptr) == RBA_OK);
                    EXPECT(rba_prefill_relproj(&p, P(), P(), P(), 64, P(), P(), 64, 1, (const int32_t*)P(),
                                               (const int32_t*)P(), (const int32_t*)P(), 64, 1, 100, 8192, nullptr,
                                               nullptr, (float*)P(), nullptr, nullptr) == RBA_OK);
                    for (int mask = 0; mask < 16; ++mask) {  // every mix of sink, gate, logit scale, e4m3
                        rba_call_options o;
                        memset(&o, 0, sizeof(o));
                        o.sink = (mask & 1) ? (const float*)P(4) : nullptr;
                        o.gate = (mask & 2) ? (const float*)P(8) : nullptr;
                        o.logit_scale = (mask & 4) ? (const float*)P(12) : nullptr;
                        o.kv_e4m3 = (mask & 8) ? 1 : 0;
                        o.k_scale = 0.5f;
                        o.v_scale = 0.25f;
                        EXPECT(rba_prefill_ex(&p, P(), P(), P(), 64, rel, (const int32_t*)P(), (const int32_t*)P(),
                                              (const int32_t*)P(), 64, 2, 300, 8192, &o, (float*)P(), (float*)P(4),
                                              nullptr) == RBA_OK);
                        EXPECT(rba_prefill_relproj_ex(&p, P(), P(), P(), 64, P(), P(), 32 << (mask & 2 ? 1 : 0), 1,
                                                      (const int32_t*)P(), (const int32_t*)P(), (const int32_t*)P(),
                                                      64, 1, 100, 8192, &o, (float*)P(), nullptr, nullptr) == RBA_OK);
                    }
                }
    rba_attn_params p = prm(32, 8, 128, 512, 512);
    // rejected arguments: nothing launched, an error code and a message
    EXPECT(rba_prefill(nullptr, P(), P(), P(), 64, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(),
                       (const int32_t*)P(), 64, 1, 8192, 8192, (float*)P(), nullptr, nullptr) == RBA_ERR_NULL);
    EXPECT(strlen(rba_last_error()) > 0);
    EXPECT(rba_prefill(&p, nullptr, P(), P(), 64, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(),
                       (const int32_t*)P(), 64, 1, 8192, 8192, (float*)P(), nullptr, nullptr) == RBA_ERR_NULL);
    EXPECT(rba_prefill(&p, P(8), P(), P(), 64, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(),
                       (const int32_t*)P(), 64, 1, 8192, 8192, (float*)P(), nullptr, nullptr) == RBA_ERR_UNSUPPORTED);
    EXPECT(rba_prefill(&p, P(), P(), P(), 64, (const float*)P(2), (const int32_t*)P(), (const int32_t*)P(),
                       (const int32_t*)P(), 64, 1, 8192, 8192, (float*)P(), nullptr, nullptr) == RBA_ERR_UNSUPPORTED);
    EXPECT(rba_prefill(&p, P(), P(), P(), 64, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(),
                       (const int32_t*)P(), 63, 1, 8192, 8192, (float*)P(), nullptr, nullptr) == RBA_ERR_SHAPE);
    EXPECT(rba_prefill(&p, P(), P(), P(), 64, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(),
                       (const int32_t*)P(), 64, 1, 8192, 0x7fffff00, (float*)P(), nullptr, nullptr) != RBA_OK);
    EXPECT(rba_prefill_relproj(&p, P(), P(), P(), 64, P(), P(), 48, 1, (const int32_t*)P(), (const int32_t*)P(),
                               (const int32_t*)P(), 64, 1, 100, 8192, nullptr, nullptr, (float*)P(), nullptr,
                               nullptr) == RBA_ERR_UNSUPPORTED);
    EXPECT(rba_prefill_relproj(&p, P(), P(), P(), 64, P(), P(), 64, 3, (const int32_t*)P(), (const int32_t*)P(),
                               (const int32_t*)P(), 64, 1, 100, 8192, nullptr, nullptr, (float*)P(), nullptr,
                               nullptr) == RBA_ERR_SHAPE);
    EXPECT(rba_prefill_logpos(&p, P(), P(), P(), 64, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(),
                              (const int32_t*)P(), 64, 1, 100, 8192, nullptr, (float*)P(), nullptr,
                              nullptr) == RBA_ERR_NULL);
    {  // options checked before anything else
        rba_call_options o;
        memset(&o, 0, sizeof(o));
        o.kv_e4m3 = 2;
        EXPECT(rba_prefill_ex(&p, P(), P(), P(), 64, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(),
                              (const int32_t*)P(), 64, 1, 8192, 8192, &o, (float*)P(), nullptr, nullptr) ==
               RBA_ERR_SHAPE);
        o.kv_e4m3 = 1;
        o.k_scale = 0.f;
        o.v_scale = 1.f;
        EXPECT(rba_prefill_ex(&p, P(), P(), P(), 64, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(),
                              (const int32_t*)P(), 64, 1, 8192, 8192, &o, (float*)P(), nullptr, nullptr) ==
               RBA_ERR_SHAPE);
        o.kv_e4m3 = 0;
        o.sink = (const float*)P(2);
        EXPECT(rba_prefill_ex(&p, P(), P(), P(), 64, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(),
                              (const int32_t*)P(), 64, 1, 8192, 8192, &o, (float*)P(), nullptr, nullptr) ==
               RBA_ERR_UNSUPPORTED);
    }
    // empty calls need no pointers
    EXPECT(rba_prefill(&p, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0, nullptr,
                       nullptr, nullptr) == RBA_OK);
}

static void decode_cases() {
    const int Hs[][2] = {{32, 8}, {64, 8}, {48, 8}, {16, 4}, {128, 8}, {8, 8}, {64, 2}};
    for (auto& h : Hs)
        for (int n_q : {1, 2, 4, 8, 16})
            for (int dv : {64, 128})
                for (int W : {0, 300})
                    for (int msl : {16, 1000, 100000, 131072}) {
                        rba_attn_params p = prm(h[0], h[1], dv, 1023, W);
                        const int G = h[0] / h[1];
                        if (G * n_q > 256 || msl < n_q) continue;
                        for (int cus : {1, 80, 256, 304}) {
                            const int32_t s = rba_decode_plan_splits(&p, 16, n_q, msl, cus);
                            EXPECT(s >= 1 && s <= 256);
                        }
                        const size_t ws = rba_decode_workspace_size(&p, 3, n_q, msl, 0);
                        EXPECT(ws > 0);
                        const int maxb = (msl + 127) / 128;
                        EXPECT(rba_decode(&p, P(), P(), P(), maxb, (const float*)P(4), (const int32_t*)P(),
                                          (const int32_t*)P(), maxb, 3, n_q, msl, 0, P(), ws, (float*)P(), nullptr,
                                          nullptr) == RBA_OK);
                        EXPECT(rba_decode(&p, P(), P(), P(), maxb, (const float*)P(4), (const int32_t*)P(),
                                          (const int32_t*)P(), maxb, 3, n_q, msl, 0, P(), ws - 1, (float*)P(),
                                          nullptr, nullptr) == RBA_ERR_WORKSPACE);
                        EXPECT(rba_decode_fp8(&p, P(), P(), P(), maxb, 0.5f, 0.25f, (const float*)P(4),
                                              (const int32_t*)P(), (const int32_t*)P(), maxb, 3, n_q, msl, 0, P(),
                                              ws, (float*)P(), nullptr, nullptr) == RBA_OK);
                        EXPECT(rba_decode_gated(&p, P(), P(), P(), maxb, (const float*)P(4), (const int32_t*)P(),
                                                (const int32_t*)P(), maxb, 3, n_q, msl, 0, P(), ws,
                                                (const float*)P(4), nullptr, (float*)P(), nullptr,
                                                nullptr) == RBA_OK);
                        EXPECT(rba_decode_logpos(&p, P(), P(), P(), maxb, (const float*)P(4), (const int32_t*)P(),
                                                 (const int32_t*)P(), maxb, 3, n_q, msl, 0, P(), ws,
                                                 (const float*)P(4), (float*)P(), nullptr, nullptr) == RBA_OK);
                        for (int mask = 0; mask < 16; ++mask) {
                            rba_call_options o;
                            memset(&o, 0, sizeof(o));
                            o.sink = (mask & 1) ? (const float*)P(4) : nullptr;
                            o.gate = (mask & 2) ? (const float*)P(8) : nullptr;
                            o.logit_scale = (mask & 4) ? (const float*)P(12) : nullptr;
                            o.kv_e4m3 = (mask & 8) ? 1 : 0;
                            o.k_scale = 0.5f;
                            o.v_scale = 0.25f;
                            EXPECT(rba_decode_ex(&p, P(), P(), P(), maxb, (const float*)P(4), (const int32_t*)P(),
                                                 (const int32_t*)P(), maxb, 3, n_q, msl, 0, P(), ws, &o, (float*)P(),
                                                 nullptr, nullptr) == RBA_OK);
                        }
                        // bias rows made from r: the workspace adds them after the partials
                        const size_t wr = rba_decode_relproj_workspace_size(&p, 3, n_q, msl, 0);
                        EXPECT(wr >= ws + (size_t)3 * n_q * p.num_heads_q * p.rel_extent * 4);
                        for (int d_r : {32, 64, 128})
                            for (int ph : {1, p.num_heads_q}) {
                                EXPECT(rba_decode_relproj(&p, P(), P(), P(), maxb, P(), P(), d_r, ph,
                                                          (const int32_t*)P(), (const int32_t*)P(), maxb, 3, n_q,
                                                          msl, 0, P(), wr, nullptr, (float*)P(), nullptr,
                                                          nullptr) == RBA_OK);
                            }
                        EXPECT(rba_decode_relproj(&p, P(), P(), P(), maxb, P(), P(), 64, 1, (const int32_t*)P(),
                                                  (const int32_t*)P(), maxb, 3, n_q, msl, 0, P(), wr - 1, nullptr,
                                                  (float*)P(), nullptr, nullptr) == RBA_ERR_WORKSPACE);
                        const size_t ws3 = rba_decode_workspace_size(&p, 3, n_q, msl, 3);
                        EXPECT(rba_decode_split(&p, P(), P(), P(), maxb, (const float*)P(4), (const int32_t*)P(),
                                                (const int32_t*)P(), maxb, 3, n_q, msl, 3, P(), ws3,
                                                nullptr) == RBA_OK);
                        EXPECT(rba_decode_combine(&p, 3, n_q, 3, P(), ws3, (float*)P(), (float*)P(4),
                                                  nullptr) == RBA_OK);
                    }
    rba_attn_params p = prm(32, 8, 128, 1024, 0);
    EXPECT(rba_decode_plan_splits(&p, 0, 1, 1000, 256) < 0);
    EXPECT(rba_decode_plan_splits(&p, 1, 1, 1000, 0) < 0);
    EXPECT(rba_decode_workspace_size(&p, 1, 0, 1000, 0) == 0);
    EXPECT(rba_decode_workspace_size(&p, 1, 1, 1000, 2000) == 0);
    EXPECT(rba_decode(&p, P(), P(), P(), 8, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(), 8, 1, 1,
                      1000, 0, nullptr, 0, (float*)P(), nullptr, nullptr) == RBA_ERR_WORKSPACE);
    EXPECT(rba_decode(&p, P(), P(), P(), 8, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(), 8, 1, 300,
                      1000, 0, P(), 1 << 30, (float*)P(), nullptr, nullptr) == RBA_ERR_UNSUPPORTED);
    EXPECT(rba_decode_split(&p, P(), P(), P(), 8, (const float*)P(), (const int32_t*)P(), (const int32_t*)P(), 8, 1,
                            1, 1000, 0, P(), 1 << 30, nullptr) == RBA_ERR_SHAPE);
    EXPECT(rba_decode_fp8(&p, P(), P(), P(), 8, 0.f, 1.f, (const float*)P(), (const int32_t*)P(),
                          (const int32_t*)P(), 8, 1, 1, 1000, 0, P(), 1 << 30, (float*)P(), nullptr,
                          nullptr) == RBA_ERR_SHAPE);
    EXPECT(rba_decode_combine(&p, 1, 1, 0, P(), 1 << 30, (float*)P(), nullptr, nullptr) == RBA_ERR_SHAPE);
    {  // the bias made from r: argument checks
        const size_t wr = rba_decode_relproj_workspace_size(&p, 1, 1, 1000, 0);
        EXPECT(wr > rba_decode_workspace_size(&p, 1, 1, 1000, 0));
        EXPECT(rba_decode_relproj_workspace_size(&p, 1, 0, 1000, 0) == 0);
        EXPECT(rba_decode_relproj(&p, P(), P(), P(), 8, P(), P(), 48, 1, (const int32_t*)P(), (const int32_t*)P(),
                                  8, 1, 1, 1000, 0, P(), wr, nullptr, (float*)P(), nullptr, nullptr) ==
               RBA_ERR_UNSUPPORTED);
        EXPECT(rba_decode_relproj(&p, P(), P(), P(), 8, P(), P(), 64, 3, (const int32_t*)P(), (const int32_t*)P(),
                                  8, 1, 1, 1000, 0, P(), wr, nullptr, (float*)P(), nullptr, nullptr) ==
               RBA_ERR_SHAPE);
        EXPECT(rba_decode_relproj(&p, P(), P(), P(), 8, nullptr, P(), 64, 1, (const int32_t*)P(),
                                  (const int32_t*)P(), 8, 1, 1, 1000, 0, P(), wr, nullptr, (float*)P(), nullptr,
                                  nullptr) == RBA_ERR_NULL);
        EXPECT(rba_decode_relproj(&p, P(), P(), P(), 8, P(), nullptr, 64, 1, (const int32_t*)P(),
                                  (const int32_t*)P(), 8, 1, 1, 1000, 0, P(), wr, nullptr, (float*)P(), nullptr,
                                  nullptr) == RBA_ERR_NULL);
        EXPECT(rba_decode_relproj(&p, P(), P(), P(), 8, P(8), P(), 64, 1, (const int32_t*)P(),
                                  (const int32_t*)P(), 8, 1, 1, 1000, 0, P(), wr, nullptr, (float*)P(), nullptr,
                                  nullptr) == RBA_ERR_UNSUPPORTED);
        rba_call_options o;
        memset(&o, 0, sizeof(o));
        o.kv_e4m3 = 1;
        o.k_scale = -1.f;
        o.v_scale = 1.f;
        EXPECT(rba_decode_relproj(&p, P(), P(), P(), 8, P(), P(), 64, 1, (const int32_t*)P(), (const int32_t*)P(),
                                  8, 1, 1, 1000, 0, P(), wr, &o, (float*)P(), nullptr, nullptr) == RBA_ERR_SHAPE);
        EXPECT(rba_decode_relproj(&p, P(), P(), P(), 8, P(), P(), 64, 1, (const int32_t*)P(), (const int32_t*)P(),
                                  8, 0, 1, 1000, 0, nullptr, 0, nullptr, nullptr, nullptr, nullptr) == RBA_OK);
    }
    {  // the split stage alone takes no sink or gate, and needs a resolved split count
        rba_call_options o;
        memset(&o, 0, sizeof(o));
        o.sink = (const float*)P(4);
        EXPECT(rba_decode_split_ex(&p, P(), P(), P(), 8, (const float*)P(), (const int32_t*)P(),
                                   (const int32_t*)P(), 8, 1, 1, 1000, 2, P(), 1 << 30, &o, nullptr) ==
               RBA_ERR_UNSUPPORTED);
        o.sink = nullptr;
        o.kv_e4m3 = 1;
        o.k_scale = o.v_scale = 1.f;
        o.logit_scale = (const float*)P(4);
        EXPECT(rba_decode_split_ex(&p, P(), P(), P(), 8, (const float*)P(), (const int32_t*)P(),
                                   (const int32_t*)P(), 8, 1, 1, 1000, 2, P(), 1 << 30, &o, nullptr) == RBA_OK);
        EXPECT(rba_decode_split_ex(&p, P(), P(), P(), 8, (const float*)P(), (const int32_t*)P(),
                                   (const int32_t*)P(), 8, 1, 1, 1000, 0, P(), 1 << 30, &o, nullptr) ==
               RBA_ERR_SHAPE);
    }
}

int main() {
    EXPECT(strncmp(rba_version(), "librba", 6) == 0);
    prefill_cases();
    decode_cases();
    // concurrent first calls fill the per-device CU cache from several threads
    std::vector<std::thread> ts;
    for (int t = 0; t < 8; ++t)
        ts.emplace_back([] {
            rba_attn_params p = prm(32, 8, 128, 1024, 0);
            for (int i = 0; i < 50; ++i) (void)rba_decode_workspace_size(&p, 16, 1, 131072, 0);
        });
    for (auto& t : ts) t.join();
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("host driver: all expectations held\n");
    return 0;
}
