// Host-only stand-ins for the kernel launchers, for the sanitizer build of
// rba_host.cpp (no GPU code is compiled or run). Each one checks the
// launch arguments the host code prepared against the invariants the
// kernels rely on and aborts if one is broken, then reports success.
#include <stdio.h>
#include <stdlib.h>

#include "rba_internal.h"

namespace rba {

static void expect(bool ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "launch invariant broken: %s\n", what);
        abort();
    }
}

hipError_t launch_prefill(const PrefillArgs& a, int dv, hipStream_t) {
    expect(dv == 64 || dv == 128, "dv");
    expect(a.q && a.k && a.v && a.cu_q && a.seq_lens && a.tables && a.out, "pointers");
    expect(a.rel != nullptr || a.r != nullptr, "bias source");
    expect(a.Hq == a.Hkv * a.G && a.G % a.hpw == 0 && a.n_hc * a.hpw == a.G, "head split");
    expect(a.QT == 32 * (8 / a.hpw) && a.n_qt >= 1 && a.batch >= 1, "tiles");
    expect(a.R >= 1 && a.W >= 0 && a.max_blocks >= 1 && a.num_blocks >= 1, "sizes");
    expect((a.kv8 == 0 && a.v_scale == 1.f) || (a.kv8 == 1 && a.v_scale > 0.f), "K/V type");
    return hipSuccess;
}

hipError_t launch_prefill_relproj(const PrefillArgs& a, int dv, hipStream_t s) {
    expect(a.r && a.proj && (a.proj_heads == 1 || a.proj_heads == a.Hq), "projection");
    expect(a.d_r == 32 || a.d_r == 64 || a.d_r == 128, "width of r");
    return launch_prefill(a, dv, s);
}

hipError_t launch_decode_split(const DecodeArgs& a, int dv, hipStream_t) {
    expect(dv == 64 || dv == 128, "dv");
    expect(a.q && a.k && a.v && a.rel && a.seq_lens && a.tables && a.part_o && a.part_lse, "pointers");
    // 33 to 64 columns over bf16 K/V run as one workgroup for both groups
    expect(a.Hq == a.Hkv * a.G && a.n_q >= 1 &&
               (a.n_cg * 32 >= a.G * a.n_q || (a.n_cg == 1 && a.kv8 == 0 && a.G * a.n_q <= 64)),
           "columns");
    expect(a.splits >= 1 && a.bps >= 1 && a.batch >= 1, "split plan");
    // the splits cover the longest visible range
    const long long nb_max = (a.max_blocks > 0) ? a.max_blocks : 0;
    expect((long long)a.splits * a.bps >= 1 && nb_max >= 1, "coverage");
    expect(a.part_lse > a.part_o, "workspace layout");
    return hipSuccess;
}

hipError_t launch_rel_rows(const RelRowsArgs& a, hipStream_t) {
    expect(a.r && a.proj && a.rel, "bias-row pointers");
    expect(a.d_r == 32 || a.d_r == 64 || a.d_r == 128, "width of r");
    expect(a.proj_heads == 1 || a.proj_heads == a.Hq, "projection heads");
    expect(a.rows >= 1 && a.Hq >= 1 && a.R >= 1, "bias-row sizes");
    expect(a.rows_per_wg >= 1 && (a.rows + a.rows_per_wg - 1) / a.rows_per_wg <= 65535, "bias-row groups");
    expect((reinterpret_cast<uintptr_t>(a.rel) & 15u) == 0, "bias-row alignment");
    return hipSuccess;
}

hipError_t launch_combine(const CombineArgs& a, int dv, hipStream_t) {
    expect(dv == 64 || dv == 128, "dv");
    expect(a.part_o && a.part_lse && a.out && a.pairs >= 1 && a.splits >= 1 && a.splits <= 1024, "combine");
    return hipSuccess;
}

}  // namespace rba

namespace rba {

// No GPU: the scratch address of the no-allocation decode is a fake,
// 256-byte aligned host value that the stand-in launchers never dereference.
hipError_t noalloc_scratch(void** ptr) {
    *ptr = reinterpret_cast<void*>(0x7f0000000000ull);
    return hipSuccess;
}

}  // namespace rba
