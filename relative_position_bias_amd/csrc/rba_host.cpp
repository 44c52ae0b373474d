// Host side of librba: argument validation, the split plan, workspace sizing
// and the C-ABI entry points declared in include/rba.h. Validation and
// planning are pure host code (no HIP call), so they can be exercised on a
// machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include <hip/hip_runtime.h>

#include "rba.h"
#include "rba_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return RBA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_params(const rba_attn_params* p) {
    if (p == nullptr) return fail(RBA_ERR_NULL, "params is NULL");
    if (p->num_heads_q < 1 || p->num_heads_kv < 1)
        return fail(RBA_ERR_SHAPE, "num_heads_q (%d) and num_heads_kv (%d) must be >= 1",
                    p->num_heads_q, p->num_heads_kv);
    if (p->num_heads_q % p->num_heads_kv != 0)
        return fail(RBA_ERR_SHAPE, "num_heads_q (%d) is not a multiple of num_heads_kv (%d)",
                    p->num_heads_q, p->num_heads_kv);
    if (p->head_dim_qk != RBA_HEAD_DIM_QK)
        return fail(RBA_ERR_UNSUPPORTED, "head_dim_qk %d unsupported (must be 128)", p->head_dim_qk);
    if (p->head_dim_v != 64 && p->head_dim_v != 128)
        return fail(RBA_ERR_UNSUPPORTED, "head_dim_v %d unsupported (64 or 128)", p->head_dim_v);
    if (p->rel_extent < 1) return fail(RBA_ERR_SHAPE, "rel_extent %d must be >= 1", p->rel_extent);
    if (p->window < 0) return fail(RBA_ERR_SHAPE, "window %d must be >= 0", p->window);
    if (!isfinite(p->scale)) return fail(RBA_ERR_SHAPE, "scale is not finite");
    if (p->block_size != RBA_BLOCK_SIZE)
        return fail(RBA_ERR_UNSUPPORTED, "block_size %d unsupported (must be 128)", p->block_size);
    return RBA_OK;
}

int check_cache(const void* k_cache, const void* v_cache, int32_t num_blocks,
                const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t max_seq_len) {
    if (k_cache == nullptr || v_cache == nullptr) return fail(RBA_ERR_NULL, "k_cache/v_cache is NULL");
    if (block_tables == nullptr) return fail(RBA_ERR_NULL, "block_tables is NULL");
    if (num_blocks < 1) return fail(RBA_ERR_SHAPE, "num_blocks %d must be >= 1", num_blocks);
    if (max_seq_len > INT32_MAX - 2 * RBA_BLOCK_SIZE)
        return fail(RBA_ERR_UNSUPPORTED, "max_seq_len %d too large", max_seq_len);
    if (max_blocks_per_seq < ceil_div(max_seq_len, RBA_BLOCK_SIZE))
        return fail(RBA_ERR_SHAPE, "max_blocks_per_seq %d < ceil(max_seq_len %d / 128)",
                    max_blocks_per_seq, max_seq_len);
    if (!aligned16(k_cache) || !aligned16(v_cache))
        return fail(RBA_ERR_UNSUPPORTED, "k_cache/v_cache must be 16-byte aligned");
    if (!aligned4(block_tables)) return fail(RBA_ERR_UNSUPPORTED, "block_tables must be 4-byte aligned");
    return RBA_OK;
}

// Query heads per prefill workgroup: the largest of 8, 4, 2, 1 dividing G.
int prefill_hpw(int G) {
    for (int h = 8; h > 1; h >>= 1)
        if (G % h == 0) return h;
    return 1;
}

// CU count of the current device, queried once per device. Any thread may
// fill an entry; every filler stores the same value, and the atomics make the
// concurrent first calls race-free.
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0) {
            (void)hipGetLastError();
            cus = 256;
        }
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

int64_t decode_nb_eff(const rba_attn_params* p, int32_t n_q, int32_t max_seq_len) {
    const int64_t nb_max = ceil_div(max_seq_len, RBA_BLOCK_SIZE);
    if (p->window == 0) return nb_max;
    const int64_t span = ceil_div((int64_t)p->window + n_q - 1, RBA_BLOCK_SIZE) + 1;
    return span < nb_max ? span : nb_max;
}

int32_t plan_splits(const rba_attn_params* p, int32_t batch, int32_t n_q, int32_t max_seq_len,
                    int32_t num_cus) {
    // Up to two decode workgroups are resident per CU. If one workgroup per
    // CU covers the longest sequence with at most 32 blocks per split, use
    // exactly that (every CU gets the same work, and the per-workgroup start
    // and merge costs are paid once per CU); this needs a variant that keeps
    // the next block's loads in flight (G * n_q <= 16, or dv <= 64), since a
    // lone workgroup otherwise has too few loads outstanding. Next, if one
    // round of two workgroups per CU covers it with at most 128 blocks per
    // split, use that round (no tail). Otherwise the lengths are long
    // compared with the machine: cut them into 32-block splits so that long
    // and short sequences spread over many workgroups. Always at least ~16
    // blocks per split and at most 256 splits.
    const int64_t G = p->num_heads_q / p->num_heads_kv;
    // 33 to 64 columns: one 8-wave workgroup covers both column groups
    // (over bf16 K/V; over e4m3 K/V the two groups run as two workgroups on
    // the same plan), one per CU, double-buffering its blocks
    const bool paired = G * n_q > 32 && G * n_q <= 64;
    const int64_t n_cg = paired ? 1 : ceil_div(G * n_q, 32);
    const int64_t nb_eff = decode_nb_eff(p, n_q, max_seq_len);
    const int64_t units = (int64_t)batch * p->num_heads_kv * n_cg;
    const bool prefetching = G * n_q <= 16 || p->head_dim_v <= 64 || paired;
    const int64_t fill1 = (int64_t)num_cus / units, fill2 = ((paired ? 1LL : 2LL) * num_cus) / units;
    int64_t want;
    if (prefetching && fill1 >= 1 && ceil_div(nb_eff, fill1) <= 32)
        want = fill1;
    else if (fill2 >= 1 && ceil_div(nb_eff, fill2) <= 128)
        want = fill2;
    else
        want = ceil_div(nb_eff, 32);
    int64_t cap = ceil_div(nb_eff, 16);
    if (cap > 256) cap = 256;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    return (int32_t)want;
}

int check_decode_shape(const rba_attn_params* p, int32_t batch, int32_t n_q, int32_t max_seq_len) {
    if (batch < 0) return fail(RBA_ERR_SHAPE, "batch %d must be >= 0", batch);
    if (n_q < 1) return fail(RBA_ERR_SHAPE, "n_q %d must be >= 1", n_q);
    const int64_t G = p->num_heads_q / p->num_heads_kv;
    if (G * n_q > 256)
        return fail(RBA_ERR_UNSUPPORTED, "G * n_q = %lld exceeds 256", (long long)(G * n_q));
    if (max_seq_len < n_q) return fail(RBA_ERR_SHAPE, "max_seq_len %d < n_q %d", max_seq_len, n_q);
    return RBA_OK;
}

size_t ws_bytes(const rba_attn_params* p, int32_t batch, int32_t n_q, int32_t splits) {
    const size_t pairs = (size_t)batch * n_q * p->num_heads_q;
    return pairs * (size_t)splits * ((size_t)p->head_dim_v + 1) * sizeof(float);
}

// rba_decode_relproj's workspace: the split partials (ws_bytes), then, from
// the next multiple of 256 bytes, the bias rows fp32 [batch*n_q, Hq, R].
size_t rel_rows_offset(const rba_attn_params* p, int32_t batch, int32_t n_q, int32_t splits) {
    return (ws_bytes(p, batch, n_q, splits) + 255) / 256 * 256;
}

size_t rel_rows_bytes(const rba_attn_params* p, int32_t batch, int32_t n_q) {
    return (size_t)batch * n_q * p->num_heads_q * (size_t)p->rel_extent * sizeof(float);
}

int check_producer(const rba_attn_params* p, const void* r, const void* rel_proj, int32_t d_r,
                   int32_t proj_heads) {
    if (d_r != 32 && d_r != 64 && d_r != 128)
        return fail(RBA_ERR_UNSUPPORTED, "d_r %d: 32, 64 or 128 are supported", d_r);
    if (proj_heads != 1 && proj_heads != p->num_heads_q)
        return fail(RBA_ERR_SHAPE, "proj_heads %d must be 1 or Hq %d", proj_heads, p->num_heads_q);
    if (rel_proj == nullptr) return fail(RBA_ERR_NULL, "rel_proj is NULL");
    if (!aligned16(r) || !aligned16(rel_proj)) return fail(RBA_ERR_UNSUPPORTED, "r/rel_proj must be 16-byte aligned");
    return RBA_OK;
}

// `rel` is the bias source the call reads (rel, or r for the in-kernel
// producer), named `rel_name` in messages.
int validate_prefill(const rba_attn_params* p, const void* q, const void* k_cache, const void* v_cache,
                     int32_t num_blocks, const void* rel, const int32_t* cu_q, const int32_t* seq_lens,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch,
                     int32_t max_q_len, int32_t max_seq_len, const float* out, const float* lse,
                     bool* nothing, const char* rel_name = "rel", bool rel_is_r = false) {
    *nothing = false;
    int rc = check_params(p);
    if (rc) return rc;
    if (batch < 0) return fail(RBA_ERR_SHAPE, "batch %d must be >= 0", batch);
    if (max_q_len < 0) return fail(RBA_ERR_SHAPE, "max_q_len %d must be >= 0", max_q_len);
    if (max_seq_len < max_q_len)
        return fail(RBA_ERR_SHAPE, "max_seq_len %d < max_q_len %d", max_seq_len, max_q_len);
    if (batch == 0 || max_q_len == 0) {
        *nothing = true;
        return ok();
    }
    if (q == nullptr || rel == nullptr || out == nullptr) return fail(RBA_ERR_NULL, "q/%s/out is NULL", rel_name);
    if (cu_q == nullptr || seq_lens == nullptr) return fail(RBA_ERR_NULL, "cu_q/seq_lens is NULL");
    rc = check_cache(k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq, max_seq_len);
    if (rc) return rc;
    if (!aligned16(q) || !aligned16(out))
        return fail(RBA_ERR_UNSUPPORTED, "q/out must be 16-byte aligned");
    // fp32 rel rows start at any multiple of R floats: 4-byte alignment; the
    // bf16 r vectors of the in-kernel producer are read 16 bytes at a time
    if (rel_is_r ? !aligned16(rel) : !aligned4(rel))
        return fail(RBA_ERR_UNSUPPORTED, "%s must be %d-byte aligned", rel_name, rel_is_r ? 16 : 4);
    if (!aligned4(cu_q) || !aligned4(seq_lens) || (lse != nullptr && !aligned4(lse)))
        return fail(RBA_ERR_UNSUPPORTED, "cu_q/seq_lens/lse must be 4-byte aligned");
    const int G = p->num_heads_q / p->num_heads_kv;
    const int hpw = prefill_hpw(G);
    const int64_t QT = 32LL * (8 / hpw);
    const int64_t grid = (int64_t)batch * ceil_div(max_q_len, QT) * p->num_heads_kv * (G / hpw);
    if (grid > INT32_MAX) return fail(RBA_ERR_UNSUPPORTED, "launch too large (%lld workgroups)", (long long)grid);
    return ok();
}

int validate_decode(const rba_attn_params* p, const void* q, const void* k_cache, const void* v_cache,
                    int32_t num_blocks, const float* rel, const int32_t* seq_lens,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch, int32_t n_q,
                    int32_t max_seq_len, int32_t num_splits, const void* workspace,
                    size_t workspace_bytes, const float* out, const float* lse, bool need_out,
                    int32_t* splits_out, bool* nothing, const char* rel_name = "rel") {
    *nothing = false;
    int rc = check_params(p);
    if (rc) return rc;
    rc = check_decode_shape(p, batch, n_q, max_seq_len);
    if (rc) return rc;
    if (num_splits < 0 || num_splits > 1024)
        return fail(RBA_ERR_SHAPE, "num_splits %d out of range [0, 1024]", num_splits);
    if (batch == 0) {
        *nothing = true;
        return ok();
    }
    if (q == nullptr || rel == nullptr || seq_lens == nullptr)
        return fail(RBA_ERR_NULL, "q/%s/seq_lens is NULL", rel_name);
    if (need_out && out == nullptr) return fail(RBA_ERR_NULL, "out is NULL");
    rc = check_cache(k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq, max_seq_len);
    if (rc) return rc;
    if (!aligned16(q) || (need_out && !aligned16(out)))
        return fail(RBA_ERR_UNSUPPORTED, "q/out must be 16-byte aligned");
    if (!aligned4(rel)) return fail(RBA_ERR_UNSUPPORTED, "%s must be 4-byte aligned", rel_name);
    if (!aligned4(seq_lens) || (lse != nullptr && !aligned4(lse)))
        return fail(RBA_ERR_UNSUPPORTED, "seq_lens/lse must be 4-byte aligned");
    const int32_t splits = num_splits ? num_splits : plan_splits(p, batch, n_q, max_seq_len, device_cus());
    const size_t need = ws_bytes(p, batch, n_q, splits);
    if (workspace == nullptr) return fail(RBA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return fail(RBA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(RBA_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    const int64_t G = p->num_heads_q / p->num_heads_kv;
    const int64_t grid = (int64_t)batch * p->num_heads_kv * ceil_div(G * n_q, 32) * splits;
    if (grid > INT32_MAX) return fail(RBA_ERR_UNSUPPORTED, "launch too large (%lld workgroups)", (long long)grid);
    if ((int64_t)batch * n_q * p->num_heads_q * splits > INT32_MAX)
        return fail(RBA_ERR_UNSUPPORTED, "too many partial rows");
    *splits_out = splits;
    return ok();
}

rba::DecodeArgs decode_args(const rba_attn_params* p, const void* q, const void* k_cache,
                            const void* v_cache, int32_t num_blocks, const float* rel,
                            const int32_t* seq_lens, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, int32_t batch, int32_t n_q, int32_t max_seq_len,
                            int32_t splits, void* workspace, bool kv8) {
    rba::DecodeArgs a;
    const int G = p->num_heads_q / p->num_heads_kv;
    const size_t pairs = (size_t)batch * n_q * p->num_heads_q;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k_cache);
    a.v = static_cast<const uint16_t*>(v_cache);
    a.rel = rel;
    a.seq_lens = seq_lens;
    a.tables = block_tables;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = static_cast<float*>(workspace) + pairs * splits * p->head_dim_v;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.batch = batch;
    a.Hq = p->num_heads_q;
    a.Hkv = p->num_heads_kv;
    a.G = G;
    a.R = p->rel_extent;
    a.W = p->window;
    a.c1 = (float)((double)p->scale * 1.4426950408889634);
    a.v_scale = 1.0f;
    a.kv8 = 0;
    a.lscale = nullptr;
    a.n_q = n_q;
    // 33 to 64 columns over bf16 K/V: one workgroup for both column groups
    a.n_cg = (!kv8 && G * n_q > 32 && G * n_q <= 64) ? 1 : (int32_t)ceil_div((int64_t)G * n_q, 32);
    a.splits = splits;
    a.bps = (int32_t)ceil_div(decode_nb_eff(p, n_q, max_seq_len), splits);
    a.wide = (int64_t)batch * a.Hkv * a.n_cg * splits <= device_cus() ? 1 : 0;
    return a;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(RBA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* rba_version(void) { return "librba 0.1.0 gfx950"; }

const char* rba_last_error(void) { return g_err; }

int rba_validate_prefill(const rba_attn_params* params, const void* q, const void* k_cache,
                         const void* v_cache, int32_t num_blocks, const float* rel, const int32_t* cu_q,
                         const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                         int32_t batch, int32_t max_q_len, int32_t max_seq_len, const float* out) {
    bool nothing;
    return validate_prefill(params, q, k_cache, v_cache, num_blocks, rel, cu_q, seq_lens, block_tables,
                            max_blocks_per_seq, batch, max_q_len, max_seq_len, out, nullptr, &nothing);
}

}  // extern "C"

namespace {

// The optional terms of a call, resolved from rba_call_options (NULL: none).
struct Opts {
    const float* sink = nullptr;
    const float* gate = nullptr;
    const float* lscale = nullptr;
    bool kv8 = false;
    float k_scale = 1.f, v_scale = 1.f;
};

int check_kv_scales(float k_scale, float v_scale) {
    if (!(k_scale > 0.f && k_scale < INFINITY) || !(v_scale > 0.f && v_scale < INFINITY))
        return fail(RBA_ERR_SHAPE, "k_scale %g / v_scale %g must be finite and > 0", (double)k_scale,
                    (double)v_scale);
    return RBA_OK;
}

int check_opts(const Opts& o) {
    if (!aligned4(o.sink) || !aligned4(o.gate) || !aligned4(o.lscale))
        return fail(RBA_ERR_UNSUPPORTED, "sink/gate/logit_scale must be 4-byte aligned");
    return o.kv8 ? check_kv_scales(o.k_scale, o.v_scale) : RBA_OK;
}

int read_options(const rba_call_options* in, Opts* o) {
    *o = Opts();
    if (in == nullptr) return RBA_OK;
    if (in->kv_e4m3 != 0 && in->kv_e4m3 != 1)
        return fail(RBA_ERR_SHAPE, "kv_e4m3 %d must be 0 or 1", in->kv_e4m3);
    o->sink = in->sink;
    o->gate = in->gate;
    o->lscale = in->logit_scale;
    o->kv8 = in->kv_e4m3 == 1;
    o->k_scale = in->k_scale;
    o->v_scale = in->v_scale;
    return RBA_OK;
}

void tile_shape(rba::PrefillArgs& a, int32_t max_q_len) {
    a.hpw = prefill_hpw(a.G);
    a.QT = 32 * (8 / a.hpw);
    a.n_qt = (int32_t)ceil_div(max_q_len, a.QT);
    a.n_hc = a.G / a.hpw;
}

int prefill_impl(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                 int32_t num_blocks, const float* rel, const int32_t* cu_q, const int32_t* seq_lens,
                 const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch, int32_t max_q_len,
                 int32_t max_seq_len, const Opts& o, float* out, float* lse, void* stream) {
    int rc = check_opts(o);
    if (rc) return rc;
    bool nothing;
    rc = validate_prefill(params, q, k_cache, v_cache, num_blocks, rel, cu_q, seq_lens, block_tables,
                          max_blocks_per_seq, batch, max_q_len, max_seq_len, out, lse, &nothing);
    if (rc || nothing) return rc;
    rba::PrefillArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k_cache);
    a.v = static_cast<const uint16_t*>(v_cache);
    a.rel = rel;
    a.r = nullptr;
    a.proj = nullptr;
    a.proj_heads = 0;
    a.d_r = 0;
    a.lscale = o.lscale;
    a.cu_q = cu_q;
    a.seq_lens = seq_lens;
    a.tables = block_tables;
    a.out = out;
    a.lse = lse;
    a.sink = o.sink;
    a.gate = o.gate;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.batch = batch;
    a.Hq = params->num_heads_q;
    a.Hkv = params->num_heads_kv;
    a.G = params->num_heads_q / params->num_heads_kv;
    a.R = params->rel_extent;
    a.W = params->window;
    a.c1 = (float)((double)params->scale * (o.kv8 ? (double)o.k_scale : 1.0) * 1.4426950408889634);
    a.kv8 = o.kv8 ? 1 : 0;
    a.v_scale = o.kv8 ? o.v_scale : 1.f;
    tile_shape(a, max_q_len);
    hipError_t e = rba::launch_prefill(a, params->head_dim_v, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return ok();
}

int relproj_impl(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                 int32_t num_blocks, const void* r, const void* rel_proj, int32_t d_r, int32_t proj_heads,
                 const int32_t* cu_q, const int32_t* seq_lens, const int32_t* block_tables,
                 int32_t max_blocks_per_seq, int32_t batch, int32_t max_q_len, int32_t max_seq_len, const Opts& o,
                 float* out, float* lse, void* stream) {
    int rc = check_opts(o);
    if (rc) return rc;
    bool nothing;
    rc = validate_prefill(params, q, k_cache, v_cache, num_blocks, r, cu_q, seq_lens, block_tables,
                          max_blocks_per_seq, batch, max_q_len, max_seq_len, out, lse, &nothing, "r", true);
    if (rc || nothing) return rc;
    rc = check_producer(params, r, rel_proj, d_r, proj_heads);
    if (rc) return rc;
    rba::PrefillArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k_cache);
    a.v = static_cast<const uint16_t*>(v_cache);
    a.rel = nullptr;
    a.r = static_cast<const uint16_t*>(r);
    a.proj = static_cast<const uint16_t*>(rel_proj);
    a.proj_heads = proj_heads;
    a.d_r = d_r;
    a.lscale = o.lscale;
    a.cu_q = cu_q;
    a.seq_lens = seq_lens;
    a.tables = block_tables;
    a.out = out;
    a.lse = lse;
    a.sink = o.sink;
    a.gate = o.gate;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.batch = batch;
    a.Hq = params->num_heads_q;
    a.Hkv = params->num_heads_kv;
    a.G = params->num_heads_q / params->num_heads_kv;
    a.R = params->rel_extent;
    a.W = params->window;
    a.c1 = (float)((double)params->scale * (o.kv8 ? (double)o.k_scale : 1.0) * 1.4426950408889634);
    a.kv8 = o.kv8 ? 1 : 0;
    a.v_scale = o.kv8 ? o.v_scale : 1.f;
    tile_shape(a, max_q_len);
    hipError_t e = rba::launch_prefill_relproj(a, params->head_dim_v, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return ok();
}

// Split stage, then (if `combine`) the merge with the sink and gate. A split
// alone needs a resolved num_splits and takes no sink or gate (they act in
// the merge). `need_lscale`: a missing logit_scale is an error (the
// dedicated log-position entry point).
int decode_impl(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                int32_t num_blocks, const float* rel, const int32_t* seq_lens, const int32_t* block_tables,
                int32_t max_blocks_per_seq, int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                void* workspace, size_t workspace_bytes, const Opts& o, bool combine, bool need_lscale, float* out,
                float* lse, void* stream, const char* name) {
    if (!combine && num_splits < 1) return fail(RBA_ERR_SHAPE, "%s needs a resolved num_splits >= 1", name);
    if (!combine && (o.sink != nullptr || o.gate != nullptr))
        return fail(RBA_ERR_UNSUPPORTED, "%s: sink and gate act in the combine (rba_decode_combine_gated)", name);
    int rc = check_opts(o);
    if (rc) return rc;
    bool nothing;
    int32_t splits = 0;
    rc = validate_decode(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables, max_blocks_per_seq,
                         batch, n_q, max_seq_len, num_splits, workspace, workspace_bytes, out, lse, combine, &splits,
                         &nothing);
    if (rc || nothing) return rc;
    if (need_lscale && o.lscale == nullptr) return fail(RBA_ERR_NULL, "logit_scale is NULL");
    rba::DecodeArgs a = decode_args(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables,
                                    max_blocks_per_seq, batch, n_q, max_seq_len, splits, workspace, o.kv8);
    if (o.kv8) {
        a.c1 = (float)((double)params->scale * (double)o.k_scale * 1.4426950408889634);
        a.v_scale = o.v_scale;
        a.kv8 = 1;
    }
    a.lscale = o.lscale;
    hipError_t e = rba::launch_decode_split(a, params->head_dim_v, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode split launch");
    if (!combine) return ok();
    return rba_decode_combine_gated(params, batch, n_q, splits, workspace, workspace_bytes, o.sink, o.gate, out,
                                    lse, stream);
}

Opts gated_opts(const float* sink, const float* gate) {
    Opts o;
    o.sink = sink;
    o.gate = gate;
    return o;
}

Opts lscale_opts(const float* logit_scale) {
    Opts o;
    o.lscale = logit_scale;
    return o;
}

Opts fp8_opts(float k_scale, float v_scale) {
    Opts o;
    o.kv8 = true;
    o.k_scale = k_scale;
    o.v_scale = v_scale;
    return o;
}

}  // namespace

extern "C" {

int rba_prefill_ex(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                   int32_t num_blocks, const float* rel, const int32_t* cu_q, const int32_t* seq_lens,
                   const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch, int32_t max_q_len,
                   int32_t max_seq_len, const rba_call_options* options, float* out, float* lse, void* stream) {
    Opts o;
    int rc = read_options(options, &o);
    if (rc) return rc;
    return prefill_impl(params, q, k_cache, v_cache, num_blocks, rel, cu_q, seq_lens, block_tables,
                        max_blocks_per_seq, batch, max_q_len, max_seq_len, o, out, lse, stream);
}

int rba_prefill_gated(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                      int32_t num_blocks, const float* rel, const int32_t* cu_q, const int32_t* seq_lens,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch, int32_t max_q_len,
                      int32_t max_seq_len, const float* sink, const float* gate, float* out, float* lse,
                      void* stream) {
    return prefill_impl(params, q, k_cache, v_cache, num_blocks, rel, cu_q, seq_lens, block_tables,
                        max_blocks_per_seq, batch, max_q_len, max_seq_len, gated_opts(sink, gate), out, lse,
                        stream);
}

int rba_prefill_logpos(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                       int32_t num_blocks, const float* rel, const int32_t* cu_q, const int32_t* seq_lens,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch, int32_t max_q_len,
                       int32_t max_seq_len, const float* logit_scale, float* out, float* lse, void* stream) {
    if (batch > 0 && max_q_len > 0 && logit_scale == nullptr) return fail(RBA_ERR_NULL, "logit_scale is NULL");
    return prefill_impl(params, q, k_cache, v_cache, num_blocks, rel, cu_q, seq_lens, block_tables,
                        max_blocks_per_seq, batch, max_q_len, max_seq_len, lscale_opts(logit_scale), out, lse,
                        stream);
}

int rba_prefill(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                int32_t num_blocks, const float* rel, const int32_t* cu_q, const int32_t* seq_lens,
                const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch, int32_t max_q_len,
                int32_t max_seq_len, float* out, float* lse, void* stream) {
    return prefill_impl(params, q, k_cache, v_cache, num_blocks, rel, cu_q, seq_lens, block_tables,
                        max_blocks_per_seq, batch, max_q_len, max_seq_len, Opts(), out, lse, stream);
}

int rba_prefill_relproj_ex(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                           int32_t num_blocks, const void* r, const void* rel_proj, int32_t d_r, int32_t proj_heads,
                           const int32_t* cu_q, const int32_t* seq_lens, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, int32_t batch, int32_t max_q_len, int32_t max_seq_len,
                           const rba_call_options* options, float* out, float* lse, void* stream) {
    Opts o;
    int rc = read_options(options, &o);
    if (rc) return rc;
    return relproj_impl(params, q, k_cache, v_cache, num_blocks, r, rel_proj, d_r, proj_heads, cu_q, seq_lens,
                        block_tables, max_blocks_per_seq, batch, max_q_len, max_seq_len, o, out, lse, stream);
}

int rba_prefill_relproj(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                        int32_t num_blocks, const void* r, const void* rel_proj, int32_t d_r, int32_t proj_heads,
                        const int32_t* cu_q, const int32_t* seq_lens, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, int32_t batch, int32_t max_q_len, int32_t max_seq_len,
                        const float* sink, const float* gate, float* out, float* lse, void* stream) {
    return relproj_impl(params, q, k_cache, v_cache, num_blocks, r, rel_proj, d_r, proj_heads, cu_q, seq_lens,
                        block_tables, max_blocks_per_seq, batch, max_q_len, max_seq_len, gated_opts(sink, gate), out,
                        lse, stream);
}

int32_t rba_decode_plan_splits(const rba_attn_params* params, int32_t batch, int32_t n_q,
                               int32_t max_seq_len, int32_t num_cus) {
    int rc = check_params(params);
    if (rc) return rc;
    rc = check_decode_shape(params, batch, n_q, max_seq_len);
    if (rc) return rc;
    if (batch < 1) return fail(RBA_ERR_SHAPE, "batch must be >= 1 to plan");
    if (num_cus < 1) return fail(RBA_ERR_SHAPE, "num_cus %d must be >= 1", num_cus);
    ok();
    return plan_splits(params, batch, n_q, max_seq_len, num_cus);
}

size_t rba_decode_workspace_size(const rba_attn_params* params, int32_t batch, int32_t n_q,
                                 int32_t max_seq_len, int32_t num_splits) {
    if (check_params(params)) return 0;
    if (check_decode_shape(params, batch, n_q, max_seq_len)) return 0;
    if (num_splits < 0 || num_splits > 1024) return 0;
    if (batch == 0) return 0;
    const int32_t splits = num_splits ? num_splits : plan_splits(params, batch, n_q, max_seq_len, device_cus());
    return ws_bytes(params, batch, n_q, splits);
}

size_t rba_decode_relproj_workspace_size(const rba_attn_params* params, int32_t batch, int32_t n_q,
                                         int32_t max_seq_len, int32_t num_splits) {
    if (check_params(params)) return 0;
    if (check_decode_shape(params, batch, n_q, max_seq_len)) return 0;
    if (num_splits < 0 || num_splits > 1024) return 0;
    if (batch == 0) return 0;
    const int32_t splits = num_splits ? num_splits : plan_splits(params, batch, n_q, max_seq_len, device_cus());
    return rel_rows_offset(params, batch, n_q, splits) + rel_rows_bytes(params, batch, n_q);
}

int rba_validate_decode(const rba_attn_params* params, const void* q, const void* k_cache,
                        const void* v_cache, int32_t num_blocks, const float* rel, const int32_t* seq_lens,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch, int32_t n_q,
                        int32_t max_seq_len, int32_t num_splits, const void* workspace,
                        size_t workspace_bytes, const float* out) {
    bool nothing;
    int32_t splits = 0;
    return validate_decode(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables,
                           max_blocks_per_seq, batch, n_q, max_seq_len, num_splits, workspace,
                           workspace_bytes, out, nullptr, true, &splits, &nothing);
}

int rba_decode_split(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                     int32_t num_blocks, const float* rel, const int32_t* seq_lens,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch, int32_t n_q,
                     int32_t max_seq_len, int32_t num_splits, void* workspace, size_t workspace_bytes,
                     void* stream) {
    return decode_impl(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables, max_blocks_per_seq,
                       batch, n_q, max_seq_len, num_splits, workspace, workspace_bytes, Opts(), false, false, nullptr,
                       nullptr, stream, "rba_decode_split");
}

int rba_decode_split_ex(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                        int32_t num_blocks, const float* rel, const int32_t* seq_lens, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, int32_t batch, int32_t n_q, int32_t max_seq_len,
                        int32_t num_splits, void* workspace, size_t workspace_bytes, const rba_call_options* options,
                        void* stream) {
    Opts o;
    int rc = read_options(options, &o);
    if (rc) return rc;
    return decode_impl(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables, max_blocks_per_seq,
                       batch, n_q, max_seq_len, num_splits, workspace, workspace_bytes, o, false, false, nullptr,
                       nullptr, stream, "rba_decode_split_ex");
}

int rba_decode_combine_gated(const rba_attn_params* params, int32_t batch, int32_t n_q, int32_t num_splits,
                             const void* workspace, size_t workspace_bytes, const float* sink, const float* gate,
                             float* out, float* lse, void* stream) {
    if (!aligned4(sink) || !aligned4(gate)) return fail(RBA_ERR_UNSUPPORTED, "sink/gate must be 4-byte aligned");
    int rc = check_params(params);
    if (rc) return rc;
    if (batch < 0 || n_q < 1) return fail(RBA_ERR_SHAPE, "batch %d / n_q %d invalid", batch, n_q);
    if (num_splits < 1 || num_splits > 1024)
        return fail(RBA_ERR_SHAPE, "num_splits %d out of range [1, 1024]", num_splits);
    if (batch == 0) return ok();
    if (out == nullptr) return fail(RBA_ERR_NULL, "out is NULL");
    const size_t need = ws_bytes(params, batch, n_q, num_splits);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(RBA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    if (!aligned16(workspace) || !aligned16(out) || (lse != nullptr && !aligned4(lse)))
        return fail(RBA_ERR_UNSUPPORTED, "workspace/out must be 16-byte aligned, lse 4-byte");
    const int64_t pairs = (int64_t)batch * n_q * params->num_heads_q;
    if (pairs > INT32_MAX - 3) return fail(RBA_ERR_UNSUPPORTED, "too many rows");
    rba::CombineArgs a;
    a.part_o = static_cast<const float*>(workspace);
    a.part_lse = static_cast<const float*>(workspace) + (size_t)pairs * num_splits * params->head_dim_v;
    a.out = out;
    a.lse = lse;
    a.sink = sink;
    a.gate = gate;
    a.pairs = (int32_t)pairs;
    a.splits = num_splits;
    hipError_t e = rba::launch_combine(a, params->head_dim_v, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return ok();
}

int rba_decode_combine(const rba_attn_params* params, int32_t batch, int32_t n_q, int32_t num_splits,
                       const void* workspace, size_t workspace_bytes, float* out, float* lse, void* stream) {
    return rba_decode_combine_gated(params, batch, n_q, num_splits, workspace, workspace_bytes, nullptr, nullptr,
                                    out, lse, stream);
}

int rba_decode(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
               int32_t num_blocks, const float* rel, const int32_t* seq_lens, const int32_t* block_tables,
               int32_t max_blocks_per_seq, int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
               void* workspace, size_t workspace_bytes, float* out, float* lse, void* stream) {
    return decode_impl(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables, max_blocks_per_seq,
                       batch, n_q, max_seq_len, num_splits, workspace, workspace_bytes, Opts(), true, false, out, lse,
                       stream, "rba_decode");
}

int rba_decode_ex(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                  int32_t num_blocks, const float* rel, const int32_t* seq_lens, const int32_t* block_tables,
                  int32_t max_blocks_per_seq, int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                  void* workspace, size_t workspace_bytes, const rba_call_options* options, float* out, float* lse,
                  void* stream) {
    Opts o;
    int rc = read_options(options, &o);
    if (rc) return rc;
    return decode_impl(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables, max_blocks_per_seq,
                       batch, n_q, max_seq_len, num_splits, workspace, workspace_bytes, o, true, false, out, lse,
                       stream, "rba_decode_ex");
}

int rba_decode_noalloc(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                       int32_t num_blocks, const float* rel, const int32_t* seq_lens, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, int32_t batch, int32_t n_q, int32_t max_seq_len,
                       int32_t num_splits, float* out, float* lse, void* stream) {
    // Validate against the scratch's size first (no HIP call), then take its
    // device address on the current device.
    alignas(256) static char placeholder;
    bool nothing;
    int32_t splits = 0;
    int rc = validate_decode(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables,
                             max_blocks_per_seq, batch, n_q, max_seq_len, num_splits, &placeholder,
                             (size_t)-1, out, lse, true, &splits, &nothing);
    if (rc || nothing) return rc;
    const size_t need = ws_bytes(params, batch, n_q, splits);
    if (need > RBA_NOALLOC_SCRATCH_BYTES)
        return fail(RBA_ERR_WORKSPACE, "the call needs %zu bytes of scratch; rba_decode_noalloc holds %zu "
                    "(use rba_decode with a workspace)", need, (size_t)RBA_NOALLOC_SCRATCH_BYTES);
    void* scratch = nullptr;
    hipError_t e = rba::noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
    rba::DecodeArgs a = decode_args(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables,
                                    max_blocks_per_seq, batch, n_q, max_seq_len, splits, scratch, false);
    hipStream_t s = static_cast<hipStream_t>(stream);
    e = rba::launch_decode_split(a, params->head_dim_v, s);
    if (e != hipSuccess) return hip_fail(e, "decode split launch");
    return rba_decode_combine(params, batch, n_q, splits, scratch, need, out, lse, stream);
}

int rba_decode_gated(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                     int32_t num_blocks, const float* rel, const int32_t* seq_lens, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, int32_t batch, int32_t n_q, int32_t max_seq_len,
                     int32_t num_splits, void* workspace, size_t workspace_bytes, const float* sink,
                     const float* gate, float* out, float* lse, void* stream) {
    return decode_impl(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables, max_blocks_per_seq,
                       batch, n_q, max_seq_len, num_splits, workspace, workspace_bytes, gated_opts(sink, gate), true,
                       false, out, lse, stream, "rba_decode_gated");
}

int rba_decode_logpos(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                      int32_t num_blocks, const float* rel, const int32_t* seq_lens, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, int32_t batch, int32_t n_q, int32_t max_seq_len,
                      int32_t num_splits, void* workspace, size_t workspace_bytes, const float* logit_scale,
                      float* out, float* lse, void* stream) {
    return decode_impl(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables, max_blocks_per_seq,
                       batch, n_q, max_seq_len, num_splits, workspace, workspace_bytes, lscale_opts(logit_scale),
                       true, true, out, lse, stream, "rba_decode_logpos");
}

int rba_decode_split_fp8(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                         int32_t num_blocks, float k_scale, float v_scale, const float* rel,
                         const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                         int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, void* stream) {
    return decode_impl(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables, max_blocks_per_seq,
                       batch, n_q, max_seq_len, num_splits, workspace, workspace_bytes, fp8_opts(k_scale, v_scale),
                       false, false, nullptr, nullptr, stream, "rba_decode_split_fp8");
}

int rba_decode_fp8(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                   int32_t num_blocks, float k_scale, float v_scale, const float* rel, const int32_t* seq_lens,
                   const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch, int32_t n_q,
                   int32_t max_seq_len, int32_t num_splits, void* workspace, size_t workspace_bytes, float* out,
                   float* lse, void* stream) {
    return decode_impl(params, q, k_cache, v_cache, num_blocks, rel, seq_lens, block_tables, max_blocks_per_seq,
                       batch, n_q, max_seq_len, num_splits, workspace, workspace_bytes, fp8_opts(k_scale, v_scale),
                       true, false, out, lse, stream, "rba_decode_fp8");
}

int rba_decode_relproj(const rba_attn_params* params, const void* q, const void* k_cache, const void* v_cache,
                       int32_t num_blocks, const void* r, const void* rel_proj, int32_t d_r, int32_t proj_heads,
                       const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                       int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits, void* workspace,
                       size_t workspace_bytes, const rba_call_options* options, float* out, float* lse,
                       void* stream) {
    // Every check (the decode's own included) runs before the first launch.
    Opts o;
    int rc = read_options(options, &o);
    if (rc) return rc;
    rc = check_opts(o);
    if (rc) return rc;
    bool nothing;
    int32_t splits = 0;
    rc = validate_decode(params, q, k_cache, v_cache, num_blocks, static_cast<const float*>(r), seq_lens,
                         block_tables, max_blocks_per_seq, batch, n_q, max_seq_len, num_splits, workspace,
                         workspace_bytes, out, lse, true, &splits, &nothing, "r");
    if (rc || nothing) return rc;
    rc = check_producer(params, r, rel_proj, d_r, proj_heads);
    if (rc) return rc;
    const size_t off = rel_rows_offset(params, batch, n_q, splits);
    const size_t need = off + rel_rows_bytes(params, batch, n_q);
    if (workspace_bytes < need)
        return fail(RBA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    if ((int64_t)params->rel_extent * params->num_heads_q * batch * n_q > ((int64_t)1 << 40) ||
        params->num_heads_q > 65535)
        return fail(RBA_ERR_UNSUPPORTED, "bias rows too large");
    rba::RelRowsArgs ra;
    ra.r = static_cast<const uint16_t*>(r);
    ra.proj = static_cast<const uint16_t*>(rel_proj);
    ra.rel = reinterpret_cast<float*>(static_cast<char*>(workspace) + off);
    ra.rows = batch * n_q;
    ra.Hq = params->num_heads_q;
    ra.R = params->rel_extent;
    ra.d_r = d_r;
    ra.proj_heads = proj_heads;
    // rows per workgroup: the fewest (a power of two) that keep the grid
    // within about three workgroups per CU, and the grid's z extent legal
    {
        const int64_t xy = ceil_div(ra.R, 256) * (int64_t)ra.Hq;
        int64_t rpw = 1;
        while (rpw < ra.rows && (xy * ceil_div(ra.rows, rpw) > 3LL * device_cus() || ceil_div(ra.rows, rpw) > 65535))
            rpw *= 2;
        ra.rows_per_wg = (int32_t)(rpw < ra.rows ? rpw : ra.rows);
    }
    hipError_t e = rba::launch_rel_rows(ra, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "bias rows launch");
    return decode_impl(params, q, k_cache, v_cache, num_blocks, ra.rel, seq_lens, block_tables, max_blocks_per_seq,
                       batch, n_q, max_seq_len, splits, workspace, workspace_bytes, o, true, false, out, lse, stream,
                       "rba_decode_relproj");
}

}  // extern "C"
