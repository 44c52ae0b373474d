// Internal interface between the host entry points (rba_host.cpp) and the
// gfx950 kernels (rba_kernels.hip). Not installed; not part of the C ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace rba {

// One prefill launch: work unit = (sequence, query tile, KV head, head chunk).
struct PrefillArgs {
    const uint16_t* q;        // bf16 [total_q, Hq, 128]
    const uint16_t* k;        // bf16 (or e4m3 bytes) [num_blocks, Hkv, 128, 128]
    const uint16_t* v;        // bf16 (or e4m3 bytes) [num_blocks, Hkv, 128, dv]
    const float* rel;         // fp32 [total_q, Hq, R]
    const int32_t* cu_q;      // [batch + 1]
    const int32_t* seq_lens;  // [batch]
    const int32_t* tables;    // [batch, max_blocks]
    float* out;               // fp32 [total_q, Hq, dv]
    float* lse;               // fp32 [total_q, Hq] or null
    const float* sink;        // fp32 [total_q, Hq] sink logits, or null (no sink)
    const float* gate;        // fp32 [total_q, Hq] gate logits, or null (no gate)
    const uint16_t* r;        // bf16 [total_q, Hq, d_r] R-branch vectors (bias made in the kernel), or null
    const uint16_t* proj;     // bf16 [proj_heads, R, d_r] rel_logits_proj (linear-weight layout)
    int32_t proj_heads;       // 1 (shared) or Hq
    int32_t d_r;              // width of r: 32, 64 or 128
    const float* lscale;      // fp32 [total_q] per-row logit scale, or null (1)
    int32_t num_blocks, max_blocks, batch;
    int32_t Hq, Hkv, G, R, W;
    float c1;                 // scale * log2(e), times the K dequantization scale for e4m3 K/V
    int32_t kv8;              // K/V cache elements: 0 = bf16, 1 = e4m3
    float v_scale;            // V dequantization scale (1 for bf16 K/V)
    int32_t hpw;              // query heads per workgroup (divides G)
    int32_t QT;               // query rows per tile = 32 * (8 / hpw)
    int32_t n_qt;             // query tiles per sequence (from the host max_q_len)
    int32_t n_hc;             // head chunks = G / hpw
};

// One split-KV decode launch: work unit = (sequence, KV head, column group, split).
struct DecodeArgs {
    const uint16_t* q;        // bf16 [batch * n_q, Hq, 128]
    const uint16_t* k;
    const uint16_t* v;
    const float* rel;         // fp32 [batch * n_q, Hq, R]
    const int32_t* seq_lens;
    const int32_t* tables;
    float* part_o;            // fp32 [batch * n_q, Hq, splits, dv]
    float* part_lse;          // fp32 [batch * n_q, Hq, splits]
    int32_t num_blocks, max_blocks, batch;
    int32_t Hq, Hkv, G, R, W;
    float c1;                 // scale * log2(e), times the K dequantization scale for e4m3 K/V
    float v_scale;            // V dequantization scale (1 for bf16 K/V)
    const float* lscale;      // fp32 [batch * n_q] per-row logit scale, or null (1)
    int32_t kv8;              // K/V cache elements: 0 = bf16, 1 = e4m3 (OCP FP8, one byte)
    int32_t n_q, n_cg, splits, bps;   // column groups of 32 (head, token) pairs; blocks per split
    int32_t wide;             // 1: the grid fits one workgroup per CU (8-wave e4m3 dv-64 variant)
};

struct CombineArgs {
    const float* part_o;
    const float* part_lse;
    float* out;
    float* lse;
    const float* sink;        // fp32 [batch * n_q, Hq] sink logits, or null
    const float* gate;        // fp32 [batch * n_q, Hq] gate logits, or null
    int32_t pairs;            // batch * n_q * Hq
    int32_t splits;
};

// Bias rows of a decode step from the R branch:
// rel[row, h, d] = sum_c r[row, h, c] * proj[hp, d, c], hp = 0 or h.
struct RelRowsArgs {
    const uint16_t* r;        // bf16 [rows, Hq, d_r]
    const uint16_t* proj;     // bf16 [proj_heads, R, d_r] (linear-weight layout)
    float* rel;               // fp32 [rows, Hq, R]
    int32_t rows, Hq, R;
    int32_t d_r;              // 32, 64 or 128
    int32_t proj_heads;       // 1 (shared) or Hq
    int32_t rows_per_wg;      // rows of one workgroup (grid z = ceil(rows / rows_per_wg) <= 65535)
};
hipError_t launch_prefill(const PrefillArgs& a, int dv, hipStream_t s);
hipError_t launch_prefill_relproj(const PrefillArgs& a, int dv, hipStream_t s);
hipError_t launch_decode_split(const DecodeArgs& a, int dv, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int dv, hipStream_t s);
hipError_t launch_rel_rows(const RelRowsArgs& a, hipStream_t s);

// The device scratch of rba_decode_noalloc: a file-scope device array of
// RBA_NOALLOC_SCRATCH_BYTES bytes in the kernels' code object, one copy per
// GPU. Its device address on the current device (looked up once per device
// with hipGetSymbolAddress, with that device current) is returned in *ptr.
hipError_t noalloc_scratch(void** ptr);

}  // namespace rba
