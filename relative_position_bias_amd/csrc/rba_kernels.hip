// gfx950 (MI355X) kernels for relative-bias grouped-query attention.
//
// Method (restated from the pages): each logit is scale * q_i . k_j plus a
// learned per-query, per-head, per-distance term rel[t, h, i - j]
// ("Inkling-Small on Gaudi 2", "Why it needed a port" and "Attention with a
// relative bias"); causal, with an optional window of W keys including the
// query's own ("Decode window"); GQA with head size 128 and a value head of
// 128 or 64 ("What was built"; "Inkling on Two DGX Sparks ...", "Wall 1").
// The bias for distances at or beyond the extent R is 0.
//
// Design (MI355X-first; the pages' FA4 / Gluon / Triton / HPU designs are
// prior art only):
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_f32_32x32x16_bf16: a wave owns 32 columns (query, head pairs) and
//     walks 32-key subtiles. Each lane then holds 16 keys of ONE column, so
//     row max / row sum are in-lane plus one exchange with lane ^ 32, and the
//     probabilities are already in the B-operand layout of the P.V MFMA.
//   * The K rows fed to the MFMA A operand are permuted (bits 2 and 3 of the
//     row index swapped) so that every lane ends up with 8 CONSECUTIVE keys per
//     16-key chunk: the lane's bias values are then contiguous in its rel row,
//     and the P.V A operand is 8 consecutive keys of one value dimension.
//   * V stays in LDS in its [key][dim] layout (the prefill rotates the
//     64-byte groups of each row against bank conflicts) and is read
//     transposed with ds_read_b64_tr_b16 (gfx950): two reads give a lane the
//     8 keys of one value dimension that the P.V MFMA needs. No shuffles, no
//     transposed writes.
//   * The bias is "sheared": element (column n, key j) needs rel[t_n, h_n,
//     i_n - j], and a lane's 8 consecutive keys are 8 consecutive (falling)
//     distances of its own rel row. The prefill stages them through a
//     per-column LDS ring (below); the decode loads, with 16-byte
//     loads, the aligned superset of its 32 rel row segments (32 rows x 36
//     floats), parks it in an LDS band and reads every lane's 16 values back
//     along the shear. Subtiles whose distances are all >= R skip rel
//     entirely; subtiles that are entirely masked (causal / window) are
//     skipped.
//   * Online softmax in fp32 in the log2 domain with a lazy reference: the
//     reference max moves only when a subtile's max exceeds it by > 16 (exact
//     rearrangement; p <= 2^16), so the rescale of the accumulator is rare.
//     The column max across the two lane halves is one v_permlane32_swap.
//   * Prefill: a workgroup of 8 waves shares each 128-key K/V block in LDS for
//     up to 8 query heads of one KV head (GQA packing) and 32..256 query rows.
//     Blocks are copied HBM -> LDS by global_load_lds into double buffers
//     (one barrier per block). The block-table slice sits in a register (one
//     entry per lane) so no load waits on a table read.
//   * Bias in the prefill: from the first 64-key stage that carries bias for
//     any row of the tile on (every stage with a window; the last ~R keys
//     without one), each wave keeps the last two 32-distance bands of its
//     columns' rel rows in a per-column LDS ring, loaded 128 bytes of a row
//     per 8 lanes, and reads each lane's values back along the shear. The
//     ring leaves room for half-block K/V stages only, so the blocks before
//     that point go whole and the rest in halves.
//   * Prefill with the bias made in the kernel (rel = r @ rel_logits_proj,
//     "Attention with a relative bias"): each wave forms the 63-distance band
//     of a subtile from r (an MFMA operand held for the whole sweep) and the
//     projection rows (from L2) with d_r / 16 more MFMAs into the same ring.
//   * e4m3 (FP8) K/V caches ("vLLM TML Inkling Support", "Future Roadmap"):
//     the decode widens each piece to bf16 in registers as it is loaded; the
//     prefill copies a block's (or stage's) bytes into a staging area of LDS
//     and widens them there, between two barriers, into the bf16 layouts its
//     compute loop reads. K's scale folds into the score scale, V's into the
//     output. Over e4m3 K the decode takes the head dimension in another
//     order, the same for q and K, so that each 16-byte load of a K row feeds
//     two score MFMAs.
//   * Decode with the bias made from r: a step's bias is only batch * n_q
//     rows, so a small separate kernel writes them into the workspace and the
//     decode kernels read them like a materialised rel.
//   * Decode: each of the 4 waves of a workgroup streams its own 32-key
//     subtile of every block of the split without any barrier: K goes straight
//     from HBM into MFMA operand registers, V into a wave-private LDS tile.
//     Each block is read once for all G * n_q columns; splits of the block
//     range go to different workgroups and a small kernel merges them by
//     log-sum-exp. With 33 to 64 columns over bf16 K/V one 8-wave workgroup
//     takes both 32-column groups and copies each block into LDS once for
//     them (prefill-style, double-buffered).
//   * Work-unit order puts the KV head in the fastest position of blockIdx so
//     that, with workgroups dealt round-robin to the 8 XCDs, all workgroups of
//     one KV head (which share its K/V) land on the same XCD and its L2.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include <atomic>

#include "rba.h"
#include "rba_internal.h"

namespace rba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BS = 128;        // keys per cache block
constexpr int DQK = 128;       // query/key head size
constexpr int RROW = 36;       // floats per LDS row of a staged rel band (36 mod 64 banks spreads 16 rows)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr float TAU = 16.0f;   // lazy-rescale threshold, log2 units (p <= 2^16)

// bf16 per LDS row of V in its natural layout. A transposed read has each
// half-wave touch 4 consecutive rows x 64 bytes; a row stride of DV + 32 bf16
// (16 mod 64 dwords for DV = 64 and 128) puts those 4 spans on disjoint banks.
template <int DV>
constexpr int vrow() { return DV + 32; }

__device__ __forceinline__ int perm32(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

// Workgroup barrier that waits only for this wave's LDS traffic: global
// prefetch loads stay in flight across it (the fence of __syncthreads would
// drain them).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// max(v, v of lane ^ 32): one v_permlane32_swap of two copies of v hands every
// lane both halves (first result: the low half's value, second: the high
// half's), a short VALU hop instead of an LDS-routed lane shuffle. The
// elements are copied to scalars before the bit casts (a bit cast of a vector
// element reads the vector's first element).
__device__ __forceinline__ float halves_max(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t lo = r[0], hi = r[1];
    return fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}

// P.V A operand from V in natural layout [key][dim] (row stride `vs` bf16):
// lane gets V[key0 + 8 (lane>>5) + 0..7][dv0 + (lane & 31)] as 8 bf16, via two
// transposed LDS reads. ds_read_b64_tr_b16 hands lane i of each 16-lane group
// the (i % 4)-th 16-bit element at the address given by lane 4k + i/4, for
// k = 0..3; the addresses below make that element V[row k][dv0 + lane & 31].
__device__ __forceinline__ bf16x8 v_operand(const __bf16* Vs, int vs, int key0, int dv0, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const __bf16* p = Vs + (key0 + 8 * (g >> 1) + (j >> 2)) * vs + dv0 + 16 * (g & 1) + 4 * (j & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * vs));
    union {
        s16x4 h[2];
        bf16x8 v;
    } u;
    u.h[0] = lo;
    u.h[1] = hi;
    return u.v;
}

// Per-wave state of 32 attention columns (one per lane & 31).
template <int DV>
struct Cols {
    bf16x8 qreg[8];        // q[col, 16 s + 8 (lane>>5) + 0..7]
    const float* relrow;   // rel row of the column (valid only if pos >= 0)
    int pos;               // absolute query position, -1 for a phantom column
    int w_lo, w_hi;        // min / max position over the wave's real columns
    bool phantom;          // some column of the wave is phantom
    f32x16 O[DV / 32];     // O^T accumulators: dv = 32 dt + 8 (r/4) + 4 (lane>>5) + r%4
    float m_ref, l_sum;    // reference max (log2 units) and partial row sum
    bool m_set;
};

// The tile tests below read only wave-uniform values (the wave index is
// taken with readfirstlane, so w_lo / w_hi / phantom live in scalar
// registers): they compile to scalar compares and branches, with no round
// trip through a vector register.

template <int DV>
__device__ __forceinline__ bool masked_all(const Cols<DV>& C, int js, int W) {
    return js > C.w_hi || (W > 0 && C.w_lo - (js + 31) >= W);
}

template <int DV>
__device__ __forceinline__ bool bias_on(const Cols<DV>& C, int js, int R) {
    return C.w_lo - (js + 31) < R;
}

// rel pieces one 32-key subtile needs for this lane's own row: row n needs
// rel[t_n, h_n, a_n .. a_n + 36) with a_n = floor4(pos_n - js - 31); lane
// (n, hh) holds the float4 pieces c4 = hh, hh + 2, ... < 9. Entries at
// distances >= R are zeros (bias 0 there), pieces below distance 0 too (those
// keys are masked). A piece wholly inside [0, R) is one 16-byte load at
// 4-byte alignment (a row starts at a multiple of R floats); the one piece
// that holds distance R - 1 when R is not a multiple of 4 is read element by
// element.
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));

struct RelRegs {
    f32x4 r[5];
};

__device__ __forceinline__ void rel_load(RelRegs& v, const float* relrow, int pos, int js, int R, int lane) {
    const int hh = lane >> 5;
    const int a_n = (pos - js - 31) & ~3;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const int c4 = hh + 2 * k;
        const int a = a_n + 4 * c4;
        v.r[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c4 < 9 && pos >= 0 && a >= 0) {
            if (a + 4 <= R) {
                v.r[k] = *reinterpret_cast<const f32x4u*>(relrow + a);
            } else if (a < R) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v.r[k][e] = a + e < R ? relrow[a + e] : 0.f;
            }
        }
    }
}

__device__ __forceinline__ void rel_store(float* Rw, const RelRegs& v, int lane) {
    const int n = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const int c4 = hh + 2 * k;
        if (c4 < 9) *reinterpret_cast<f32x4*>(Rw + n * RROW + 4 * c4) = v.r[k];
    }
}

// Start of this lane's bias values in its staged LDS row: bias for register r
// (key js + 16 (r/8) + 8 hh + r%8) is rb[16 (1 - r/8) + 7 - r%8].
__device__ __forceinline__ const float* rel_row_ptr(const float* Rw, int pos, int lane) {
    const int n = lane & 31, hh = lane >> 5;
    return Rw + n * RROW + (8 + ((pos + 1) & 3) - 8 * hh);
}

// S^T for one 32-key subtile whose K operand is already in registers.
__device__ __forceinline__ f32x16 qk_regs(const bf16x8 (&kreg)[8], const bf16x8 (&qreg)[8]) {
    f32x16 s = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st) s = mfma32(kreg[st], qreg[st], s);
    return s;
}

// Softmax of one 32-key subtile starting at key js, in three steps so that
// several column tiles can be interleaved:
//   sm_scores  x = log2-domain logits relative to the reference max (bias and
//              masks applied); returns the column's subtile max (both halves).
//   sm_rescale moves the reference max of columns whose subtile max exceeds
//              it by more than TAU (or that see their first key), rescaling
//              the accumulator; callers skip it when no lane needs it.
//   sm_probs   p = exp2(x), row sums, and the bf16 B operands of P.V.
// `s` holds S^T (lane: keys js + 16 (r/8) + 8 (lane>>5) + r%8 of column
// lane & 31); if `has_bias`, `rb` is the lane's staged bias row.
template <int DV>
__device__ __forceinline__ float sm_scores(const Cols<DV>& C, const f32x16& s, bool has_bias, const float* rb,
                                           bool need_mask, int js, int W, float c1, float l2e, int lane,
                                           float (&x)[16]) {
    const int hh = lane >> 5;
    if (has_bias) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            x[r] = fmaf(s[r], c1, fmaf(rb[16 * (1 - (r >> 3)) + 7 - (r & 7)], l2e, -C.m_ref));
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fmaf(s[r], c1, -C.m_ref);
    }
    if (need_mask) {
        const int d0 = C.pos - (js + 8 * hh);  // distance of register 0's key
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = d0 - (16 * (r >> 3) + (r & 7));
            const bool vis = d >= 0 && (W == 0 || d < W) && C.pos >= 0;
            x[r] = vis ? x[r] : -INFINITY;
        }
    }
    float M = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) M = fmaxf(M, x[r]);
    return halves_max(M);
}

template <int DV>
__device__ __forceinline__ bool sm_trigger(const Cols<DV>& C, float M) {
    return (M > TAU) || (!C.m_set && M > -INFINITY);
}

// First visible keys of a column: take their max as the reference. The
// accumulator and row sum are still zero, so nothing needs rescaling.
template <int DV>
__device__ __forceinline__ void sm_init_ref(Cols<DV>& C, float& M, float (&x)[16]) {
    if (!C.m_set && M > -INFINITY) {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] -= M;
        C.m_ref += M;
        C.m_set = true;
        M = 0.f;
    }
}

template <int DV>
__device__ __forceinline__ void sm_rescale(Cols<DV>& C, float M, float (&x)[16]) {
    const bool trig = sm_trigger(C, M);
    const float delta = trig ? M : 0.f;
    const float alpha = trig ? (C.m_set ? __builtin_amdgcn_exp2f(-delta) : 0.f) : 1.f;
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt) C.O[dt] *= alpha;
    C.l_sum *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] -= delta;
    C.m_ref += delta;
    C.m_set = C.m_set || trig;
}

template <int DV>
__device__ __forceinline__ void sm_probs(Cols<DV>& C, const float (&x)[16], bf16x8 (&pb)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(x[8 * c + i]);
            C.l_sum += p;
            pb[c][i] = (__bf16)p;
        }
    }
}

// p = exp2(x) and the bf16 B operands of P.V, without touching the row sum;
// returns the sum of the lane's 16 probabilities.
__device__ __forceinline__ float sm_probs_sum(const float (&x)[16], bf16x8 (&pb)[2]) {
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(x[8 * c + i]);
            sum += p;
            pb[c][i] = (__bf16)p;
        }
    }
    return sum;
}

// A lane whose 16 probabilities sum to at most this has none above 2^TAU
// (the sum is at least its largest term, up to fp32 rounding of 16 terms).
constexpr float PSUM_TRIGGER = 65536.f * 0.999f;

template <int DV>
__device__ __forceinline__ bool need_mask_of(const Cols<DV>& C, int js, int W) {
    return C.phantom || (js + 31 > C.w_lo) || (W > 0 && C.w_hi - js >= W);
}

// Single-tile softmax and P.V for one subtile; `vread(dt, c)` returns the P.V
// A operand: V^T rows 32 dt + (lane & 31), keys 16 c + 8 (lane>>5) .. +8.
template <int DV, class VRead>
__device__ __forceinline__ void softmax_pv(Cols<DV>& C, const f32x16& s, bool has_bias, const float* rb,
                                           int js, int W, float c1, float l2e, int lane, VRead vread) {
    float x[16];
    float M = sm_scores(C, s, has_bias, rb, need_mask_of(C, js, W), js, W, c1, l2e, lane, x);
    if (__any(!C.m_set || sm_trigger(C, M))) {
        if (__any(!C.m_set)) sm_init_ref(C, M, x);
        if (__any(sm_trigger(C, M))) sm_rescale(C, M, x);
    }
    bf16x8 pb[2];
    sm_probs(C, x, pb);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int dt = 0; dt < DV / 32; ++dt) C.O[dt] = mfma32(vread(dt, c), pb[c], C.O[dt]);
    }
}

// The lane's query operands. A column past the last real one points at a
// real row (its logits are masked and its output is never stored), so the
// loads need no branch, and no wait is forced on them before the loads that
// follow.
template <int DV>
__device__ __forceinline__ void load_q(Cols<DV>& C, const uint16_t* qrow, int lane) {
    const int hh = lane >> 5;
#pragma unroll
    for (int st = 0; st < 8; ++st) C.qreg[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st + 8 * hh);
}

// load_q in the dimension order of load_k_sub8 (e4m3 K)
template <int DV>
__device__ __forceinline__ void load_q8(Cols<DV>& C, const uint16_t* qrow, int lane) {
    const int hh = lane >> 5;
#pragma unroll
    for (int st = 0; st < 8; ++st) C.qreg[st] = *reinterpret_cast<const bf16x8*>(qrow + 32 * (st >> 1) + 16 * hh + 8 * (st & 1));
}

template <int DV>
__device__ __forceinline__ void init_acc(Cols<DV>& C) {
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt) C.O[dt] = zero16();
    C.m_ref = 0.f;
    C.l_sum = 0.f;
    C.m_set = false;
}

// Write the normalised output (and lse) of a finished wave: lane holds
// dv = 32 dt + 8 q4 + 4 hh + k of column lane & 31. `sink` (natural-log
// units, -inf for none) joins the softmax normaliser with a zero value;
// `gate` scales the output by 1 / (1 + e^-gate) (+inf for none).
template <int DV>
__device__ __forceinline__ void store_out(const Cols<DV>& C, float* orow, float* lse, bool bad, float sink,
                                          float gate, int lane, float vscale = 1.f) {
    float l_tot = C.l_sum + xor32(C.l_sum);
    float mref = C.m_ref, o_fac = 1.f;
    if (sink > -INFINITY) {  // move the reference to max(reference, sink) and add the sink's term
        const float s2 = sink * LOG2E, mn = fmaxf(mref, s2);
        o_fac = __builtin_amdgcn_exp2f(mref - mn);
        l_tot = l_tot * o_fac + __builtin_amdgcn_exp2f(s2 - mn);
        mref = mn;
    }
    const float g = gate < INFINITY ? 1.f / (1.f + __builtin_amdgcn_exp2f(-gate * LOG2E)) : 1.f;
    const float inv = bad ? NAN : o_fac / l_tot * g * vscale;
    const int hh = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = C.O[dt][4 * q4 + k] * inv;
            *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * q4 + 4 * hh) = o;
        }
    }
    if (lse != nullptr && hh == 0) *lse = bad ? NAN : (mref + __log2f(l_tot)) * LN2;
}

// e4m3 (OCP FP8) K/V. A cache element is one byte. Every e4m3 value (3
// mantissa bits, exponents 2^-9 .. 2^8) is exact in bf16, so widening to bf16
// loses nothing and the MFMAs see exactly the stored values. The
// dequantization scales are folded into the score scale (K) and the split
// outputs (V).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 8 e4m3 values (lowest address first) as 8 bf16: gfx950's
// v_cvt_scalef32_pk_bf16_fp8 widens two e4m3 values (the low or the high
// 16 bits of a register) straight to two bf16, here with scale 1 (exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(const u32x2& w) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
    bf16x8 r;
    r[0] = a[0];
    r[1] = a[1];
    r[2] = b[0];
    r[3] = b[1];
    r[4] = c[0];
    r[5] = c[1];
    r[6] = d[0];
    r[7] = d[1];
    return r;
}

// ---------------------------------------------------------------------------
// Prefill
// ---------------------------------------------------------------------------

// K/V staging. Each 128-key block is copied from HBM straight into LDS with
// global_load_lds (no register staging): every wave instruction fills 1 KB of
// LDS, lane l landing at byte 16 l, and the lanes pick their source chunks so
// that the LDS image has the layout the readers want.
//   K: 128 rows x 256 bytes, no padding. Row r holds key (r & ~31) |
//      perm32(r & 31); its logical 16-byte chunk c sits at chunk c ^ (r & 15),
//      so the 16 rows read by one half of an MFMA operand load fall on
//      distinct banks.
//   V: [key][dv], 2 DV bytes per row, no padding, read transposed. The
//      64-byte groups of a row are rotated by rot(r) = r & 3 (DV 128) or
//      (r >> 1) & 1 (DV 64): logical group G sits at (G + rot(r)) mod
//      (DV / 32), so the 4 consecutive rows one transposed read touches
//      fall on distinct banks. Rows at or past the end of the sequence are
//      copied from a 16-byte zero chunk.
// Both are double-buffered.
__device__ const u32x4 kZeroChunk = {0u, 0u, 0u, 0u};

template <int DV>
__device__ __forceinline__ int vrot(int r) {
    return DV == 128 ? (r & 3) : ((r >> 1) & 1);
}

// P.V A operand from the rotated V: lane gets V[key0 + 8 (lane>>5) + 0..7]
// [32 dt + (lane & 31)] (as v_operand), `vb` being the lane's offset for
// this dt (row and group rotation folded in) and Vsub the key0 row.
__device__ __forceinline__ bf16x8 v_operand_rot(const __bf16* Vsub, int vb, int dv) {
    const __bf16* p = Vsub + vb;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * dv));
    union {
        s16x4 h[2];
        bf16x8 v;
    } u;
    u.h[0] = lo;
    u.h[1] = hi;
    return u.v;
}

// One wave instruction of global_load_lds_dwordx4: lane l copies 16 bytes
// from `src` to LDS byte `lds + 16 l` (lds is wave-uniform). Issued as inline
// assembly, so the compiler neither tracks it nor adds waits for it: the
// kernel waits for its copies itself (vm_wait_all) before the barrier that
// publishes them.
__device__ __forceinline__ void dma16(const void* src, const void* lds) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}

// The copies are issued by the first NW waves (NW = 8 or 4), 32 / NW K and
// 2 DV / (8 NW) V instructions each (for ROWS = 128). Waves w and w + 4 share
// a SIMD and the lower one is served first, so it reaches the barrier early;
// with NW = 4 the early waves issue all copies there, which balances the
// pair. ROWS (128 or 64) rows are copied, from kblk / vblk on: a whole block
// or half of one, in the same per-row layout.
template <int DV, int NW, int ROWS = BS>
__device__ __forceinline__ void kv_dma(__bf16* Ks, __bf16* Vs, const uint16_t* kblk, const uint16_t* vblk,
                                       int nvalid, int wid, int lane) {
    if (wid >= NW) return;
#pragma unroll
    for (int i = 0; i < ROWS / (4 * NW); ++i) {
        const int grp = wid + NW * i;  // 1 KB group: K rows 4 grp .. 4 grp + 3
        const int r = 4 * grp + (lane >> 4);
        const int key = (r & ~31) | perm32(r & 31);
        const int c = (lane & 15) ^ (r & 15);
        dma16(kblk + key * DQK + 8 * c, Ks + grp * 4 * DQK);
    }
    constexpr int VCH = DV / 8, RPG = 64 / VCH;  // 16-byte chunks per V row, V rows per group
#pragma unroll
    for (int i = 0; i < ROWS / (RPG * NW); ++i) {
        const int grp = wid + NW * i;
        const int r = RPG * grp + lane / VCH;
        const int p = lane % VCH;  // physical chunk; its logical chunk undoes the group rotation
        const int c = 4 * (((p >> 2) - vrot<DV>(r)) & (DV / 32 - 1)) + (p & 3);
        const void* src = r < nvalid ? static_cast<const void*>(vblk + r * DV + 8 * c) : &kZeroChunk;
        dma16(src, Vs + grp * RPG * DV);
    }
}

// Waits until every global load this wave issued (LDS copies included) has
// landed.
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// e4m3 K/V for the prefill: the bytes of ROWS keys (a block or half of one)
// are copied into a staging area in their natural layout (K rows of 128
// bytes, then V rows of DV bytes), by the first NW waves, 1 KB per
// instruction ...
template <int DV, int NW, int ROWS = BS>
__device__ __forceinline__ void kv8_dma(uint8_t* S8, const uint8_t* kblk, const uint8_t* vblk, int wid, int lane) {
    if (wid >= NW) return;
    constexpr int KI = ROWS * DQK / 1024, VI = ROWS * DV / 1024;
#pragma unroll
    for (int i = 0; i < (KI + VI + NW - 1) / NW; ++i) {
        const int grp = wid + NW * i;  // wave-uniform
        if (grp < KI)
            dma16(kblk + grp * 1024 + 16 * lane, S8 + grp * 1024);
        else if (grp < KI + VI)
            dma16(vblk + (grp - KI) * 1024 + 16 * lane, S8 + grp * 1024);
    }
}

// ... and then widened by all 512 threads into the bf16 K/V layouts the
// readers use (the swizzled K rows and rotated V groups that kv_dma builds);
// V rows at or past the end of the sequence become zeros.
template <int DV, int ROWS = BS>
__device__ __forceinline__ void kv8_widen(__bf16* Ks, __bf16* Vs, const uint8_t* S8, int nvalid, int tid) {
#pragma unroll
    for (int i = 0; i < ROWS * DQK / 8 / 512; ++i) {
        const int u = tid + 512 * i;
        const int key = u >> 4, c = u & 15;  // key, logical 8-value chunk
        const u32x2 w = *reinterpret_cast<const u32x2*>(S8 + key * DQK + 8 * c);
        const int row = (key & ~31) | perm32(key & 31);
        *reinterpret_cast<bf16x8*>(Ks + row * DQK + 8 * (c ^ (row & 15))) = fp8x8_to_bf16(w);
    }
    constexpr int VC = DV / 8;
#pragma unroll
    for (int i = 0; i < ROWS * DV / 8 / 512; ++i) {
        const int u = tid + 512 * i;
        const int r = u / VC, c = u % VC;
        const u32x2 w = *reinterpret_cast<const u32x2*>(S8 + ROWS * DQK + r * DV + 8 * c);
        const bf16x8 x = r < nvalid ? fp8x8_to_bf16(w) : fp8x8_to_bf16(u32x2{0u, 0u});
        const int p = 4 * (((c >> 2) + vrot<DV>(r)) & (DV / 32 - 1)) + (c & 3);
        *reinterpret_cast<bf16x8*>(Vs + r * DV + 8 * p) = x;
    }
}

// S^T for one 32-key subtile of the chunk-swizzled K (koff: the lane's offset
// of operand st, row (lane & 31), logical chunk 2 st + (lane >> 5)).
__device__ __forceinline__ f32x16 qk_swz(const __bf16* Ksub, const int (&koff)[8], const bf16x8 (&qreg)[8]) {
    f32x16 s = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st) s = mfma32(*reinterpret_cast<const bf16x8*>(Ksub + koff[st]), qreg[st], s);
    return s;
}

// The bias of one subtile straight from HBM into registers: register r (key
// js + 16 (r/8) + 8 (lane>>5) + r%8) gets rel at distance pos - key. `inside`
// (wave-uniform): every distance of every lane lies in [0, R) and no lane is
// a phantom column; then each 8-key run is two 16-byte loads at 4-byte
// alignment. Otherwise every element is loaded on its own from a clamped
// index; rel_bias zeroes those at distances >= R (negative ones are masked).
struct RelVals {
    float v[16];
};

__device__ __forceinline__ void rel_fetch(RelVals& rv, const float* relrow, int pos, int js, int R, bool inside,
                                          int lane) {
    const int hh = lane >> 5;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int a = pos - js - 8 * hh - 16 * c - 7;
        if (inside) {
            const f32x4u lo = *reinterpret_cast<const f32x4u*>(relrow + a);
            const f32x4u hi = *reinterpret_cast<const f32x4u*>(relrow + a + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rv.v[8 * c + 7 - i] = lo[i];
                rv.v[8 * c + 3 - i] = hi[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) rv.v[8 * c + 7 - i] = relrow[min(max(a + i, 0), R - 1)];
        }
    }
}

__device__ __forceinline__ float rel_bias(const RelVals& rv, int r, int pos, int js, int R, bool inside, int lane) {
    if (inside) return rv.v[r];
    const int d = pos - js - 8 * (lane >> 5) - 16 * (r >> 3) - (r & 7);
    return d < R ? rv.v[r] : 0.f;
}

// The column's max over both lane halves.
__device__ __forceinline__ float sm_colmax(const float (&x)[16]) {
    float M = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) M = fmaxf(M, x[r]);
    return halves_max(M);
}

// The logits of sm_scores with the bias taken from registers (no max).
template <int DV>
__device__ __forceinline__ void sm_logits_rv(const Cols<DV>& C, const f32x16& s, bool has_bias, const RelVals& rv,
                                             bool inside, bool need_mask, int js, int W, int R, float c1, float l2e,
                                             int lane, float (&x)[16]) {
    if (has_bias) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            x[r] = fmaf(s[r], c1, fmaf(rel_bias(rv, r, C.pos, js, R, inside, lane), l2e, -C.m_ref));
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fmaf(s[r], c1, -C.m_ref);
    }
    if (need_mask) {
        const int d0 = C.pos - (js + 8 * (lane >> 5));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = d0 - (16 * (r >> 3) + (r & 7));
            const bool vis = d >= 0 && (W == 0 || d < W) && C.pos >= 0;
            x[r] = vis ? x[r] : -INFINITY;
        }
    }
}

// sm_scores with the bias taken from registers.
template <int DV>
__device__ __forceinline__ float sm_scores_rv(const Cols<DV>& C, const f32x16& s, bool has_bias, const RelVals& rv,
                                              bool inside, bool need_mask, int js, int W, int R, float c1, float l2e,
                                              int lane, float (&x)[16]) {
    sm_logits_rv(C, s, has_bias, rv, inside, need_mask, js, W, R, c1, l2e, lane, x);
    return sm_colmax(x);
}

// ---------------------------------------------------------------------------
// Prefill: the bias through a per-column band ring
//
// A wave's 32 columns are 32 consecutive positions w_lo + n of one head, so
// for the 32 keys js .. js + 31 of a subtile column n needs the distances
// (w_lo - js) + n - 31 .. (w_lo - js) + n: 63 distinct distances across the
// wave, sheared by n. Per subtile the wave puts a band T(js)[rho, n], the
// bias of column n at distance (w_lo - js) - 32 + rho for rho = 0..31, into a
// per-column ring of 64 distances that also holds T(js - 32) (the distances
// (w_lo - js) .. + 31). The shear is undone on the way out: each lane reads
// its 16 bias values as two runs of 8 consecutive ring entries starting at a
// lane-dependent slot. Ring slot of distance d at subtile js:
// (d - (w_lo - js) + 32 + 32 par(js)) mod 64, par(js) = (js / 32) mod 2;
// T(js) occupies slots 32 par .. 32 par + 31; slots 0..7 are duplicated at
// 64..71 so that no run wraps.
//
// Two band sources. Over a materialised rel (DR = 0) the band is rel entries
// that start at the same distance in every column's row: eight lanes load
// one row's 128 bytes, so one load instruction covers 8 rows (loading each
// lane's own 8-distance runs straight from HBM instead spreads every
// instruction over 32 rows, and where every subtile streams bias the vector
// memory path then saturates on the number of rows in flight). With the bias
// made in the kernel (rel = r @ rel_logits_proj, "Attention with a relative
// bias"; DR = 32, 64 or 128) the wave computes T(js)[rho, n] =
// r_n . proj[(w_lo - js) - 32 + rho] with DR / 16 32x32x16 MFMAs, r_n held
// as an MFMA operand for the whole sweep and the projection rows read from
// L2.
//
// The ring (32 x 76 floats per wave, 76 KiB for 8 waves) does not fit beside
// double-buffered whole K/V blocks, so K/V move in half blocks of 64 keys
// (two subtiles per barrier) wherever bias is in use.
// ---------------------------------------------------------------------------
constexpr int RSTRIDE = 76;  // floats per column in the band ring (64 + 8 duplicated + 4 pad)

// What a band is made from: projection rows (the A operand of the band MFMAs)
// or, for DR = 0, four 4-distance pieces of rel rows.
template <int DR>
struct BandSrc {
    bf16x8 p[DR / 16];
};
template <>
struct BandSrc<0> {
    f32x4 p[4];
};

// DR: the width of r (32, 64 or 128), or 0 for a materialised rel. LS: each
// query row's logits are multiplied by A.lscale[row] (the log-position scale
// of global layers, "What was built"); otherwise by 1. KV8: e4m3 K/V caches:
// each stage's (or whole block's) bytes are copied into a staging area of
// LDS, the copy of the next one overlapping the current compute, and widened
// between two barriers into a single pair of bf16 buffers; the compute loop
// is the bf16 one. The K scale is folded into c1, the V scale into the
// output.
//
// WB (no window): the blocks before the first subtile that carries bias for
// any row of the tile are walked whole (128-key blocks, no bias code); the
// ring and the half-block stages take over from the first block with bias.
// One LDS area is laid out twice. bf16 K/V: two
// whole-block buffers, between which the whole blocks alternate so that the
// last one is in buffer 1; the ring phase then puts its stages in buffer 0
// and the rings in buffer 1 and the LDS after it. e4m3 K/V: one bf16
// whole-block buffer and the byte staging area; the ring phase widens its
// stages into the bottom of the buffer and puts three (dv 64: two) rings
// above them, the others after the staging area.
template <int DV, bool LS, int DR, bool KV8 = false, bool WB = false>
__device__ __forceinline__ void prefill_ring_body(const PrefillArgs A) {
    constexpr int NW = WB ? 8 : 4;  // waves that issue the stage copies (measured per kernel)
    constexpr int HB = 64;  // keys per K/V stage (half a block)
    constexpr int SPB = BS / HB;
    constexpr int RING_W = 32 * RSTRIDE;        // floats of one wave's ring
    constexpr int RINGB = 4 * RING_W;           // bytes of one wave's ring
    constexpr int WHOLEB = 2 * BS * (DQK + DV); // bytes of a bf16 whole-block K/V pair
    constexpr int HALFB = 2 * HB * (DQK + DV);  // bytes of a bf16 half-block K/V pair
    constexpr int S8B = BS * (DQK + DV);        // bytes of an e4m3 whole block
    constexpr int RINGS_IN = KV8 ? (WHOLEB - HALFB) / RINGB : WHOLEB / RINGB;  // rings inside the block area
    constexpr int WB_BYTES = (KV8 ? WHOLEB + S8B : 2 * WHOLEB) + (8 - RINGS_IN) * RINGB;
    __shared__ __attribute__((aligned(16))) __bf16 K0[WB ? 8 : HB * DQK];
    __shared__ __attribute__((aligned(16))) __bf16 K1[KV8 || WB ? 8 : HB * DQK];
    __shared__ __attribute__((aligned(16))) __bf16 V0[WB ? 8 : HB * DV];
    __shared__ __attribute__((aligned(16))) __bf16 V1[KV8 || WB ? 8 : HB * DV];
    __shared__ __attribute__((aligned(16))) uint8_t S8[KV8 && !WB ? HB * (DQK + DV) : 16];
    __shared__ __attribute__((aligned(16))) float ring_all[WB ? 4 : 8 * RING_W];
    __shared__ __attribute__((aligned(16))) char WBL[WB ? WB_BYTES : 16];
    const uint8_t* const k8 = reinterpret_cast<const uint8_t*>(A.k);
    const uint8_t* const v8 = reinterpret_cast<const uint8_t*>(A.v);

    const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 31;
    const int hh = lane >> 5;
    int id = blockIdx.x;
    const int g = id % A.Hkv;
    id /= A.Hkv;
    const int b = id % A.batch;
    id /= A.batch;
    const int hc = id % A.n_hc;
    id /= A.n_hc;
    // Without a window the late tiles (more keys) go first. With one every
    // tile past the first window has the same work, and ascending order
    // measured faster for the in-kernel-bias kernel (equal for the other).
    const int qt = A.W > 0 ? id : A.n_qt - 1 - id;

    const int q_start = A.cu_q[b];
    const int q_len = A.cu_q[b + 1] - q_start;
    const int L = A.seq_lens[b];
    const int q0 = qt * A.QT;
    if (q0 >= q_len) return;  // uniform over the workgroup
    const int ctx = L - q_len;

    const int hl = hc * A.hpw + wid % A.hpw;
    const int h = g * A.G + hl;
    const int qa = q0 + (wid / A.hpw) * 32;
    const int qb = min(qa + 32, q_len) - 1;
    const bool wave_active = qa < q_len;
    const int r = qa + n;
    const bool real = r < q_len;
    const long long trow = (long long)(q_start + (real ? r : 0)) * A.Hq + h;
    const float fls = (LS && real) ? A.lscale[q_start + r] : 1.f;  // the row's logit scale
    const float c1f = A.c1 * fls, l2f = LOG2E * fls;

    Cols<DV> C;
    C.pos = real ? ctx + r : -1;
    C.relrow = nullptr;
    C.w_lo = ctx + qa;
    C.w_hi = ctx + qb;
    C.phantom = qb < qa + 31;
    const uint16_t* proj = DR > 0 ? A.proj + (size_t)(A.proj_heads == A.Hq ? h : 0) * A.R * DR : nullptr;
    // stage buffers, e4m3 staging and this wave's ring (WB: set below)
    __bf16 *Ks0 = K0, *Vs0 = V0, *Ks1 = KV8 ? K0 : K1, *Vs1 = KV8 ? V0 : V1;
    uint8_t* S8p = S8;
    float* ringw = ring_all + wid * RING_W;
    float* ring = ringw + n * RSTRIDE;  // this lane's column
    // DR = 0: rel row of the wave's first column (band pieces add the rows of
    // columns (lane >> 3) + 8 k)
    const long long rel_rs = (long long)A.Hq * A.R;
    const float* rel0 = DR == 0 && wave_active ? A.rel + ((long long)(q_start + qa) * A.Hq + h) * A.R : nullptr;

    const int i_lo = ctx + q0, i_hi = ctx + min(q0 + A.QT, q_len) - 1;
    const int s_lo = (A.W > 0 ? max(0, i_lo - A.W + 1) : 0) / HB;
    const int s_hi = i_hi / HB;
    const int kb_lo = s_lo / SPB, kb_hi = s_hi / SPB;
    // WB: whole blocks kb_lo .. kb_sw - 1, then stages from s_first. Subtile
    // js carries bias for some row of the tile iff it does for the tile's
    // first row i_lo (the others lie further from it): iff i_lo - (js + 31) < R.
    int kb_sw = kb_lo;
    if constexpr (WB) {
        const int t = i_lo - 31 - A.R;
        const int js_b = t < 0 ? 0 : (t / 32 + 1) * 32;
        kb_sw = min(max(js_b / BS, kb_lo), kb_hi + 1);
    }
    const int n1 = kb_sw - kb_lo;          // whole blocks
    const int s_first = WB ? kb_sw * SPB : s_lo;
    const int js_lo = s_first * HB;        // first key of the ring phase
    const bool ring_phase = s_first <= s_hi;
    const int* tab = A.tables + (long long)b * A.max_blocks;

    auto rel_active = [&](int js) { return wave_active && !masked_all(C, js, A.W) && bias_on(C, js, A.R); };

    // Sources of band T(jb). DR > 0: projection rows as the A operand, lane
    // row a holding the weights of distance (w_lo - jb) - 32 + a. DR = 0:
    // piece k of lane l is column 8 k + (l >> 3), distances (w_lo - jb) - 32
    // + 4 (l & 7) + 0..3. Zero outside [0, R) and for phantom columns.
    auto load_p = [&](BandSrc<DR>& pv, int jb) {
        if constexpr (DR > 0) {
            const int d = C.w_lo - jb - 32 + n;
            const bool in = (unsigned)d < (unsigned)A.R;
            const uint16_t* src = proj + (size_t)(in ? d : 0) * DR + 8 * hh;
#pragma unroll
            for (int st = 0; st < DR / 16; ++st) {
                if (in) {
                    pv.p[st] = *reinterpret_cast<const bf16x8*>(src + 16 * st);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) pv.p[st][i] = (__bf16)0.f;
                }
            }
        } else {
            const float* relc = rel0 + (lane >> 3) * rel_rs;
            const int d0 = C.w_lo - jb - 32;
            const int d = d0 + 4 * (lane & 7);
            // wave-uniform: every column real and every distance in [0, R)
            if (!C.phantom && d0 >= 0 && d0 + 31 < A.R) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const f32x4u v = *reinterpret_cast<const f32x4u*>(relc + 8 * k * rel_rs + d);
                    pv.p[k] = f32x4{v[0], v[1], v[2], v[3]};
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const bool col = 8 * k + (lane >> 3) <= qb - qa;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool in = col && (unsigned)(d + i) < (unsigned)A.R;
                        pv.p[k][i] = in ? relc[8 * k * rel_rs + d + i] : 0.f;
                    }
                }
            }
        }
    };

    // The start issues every independent load at once (q, r, the first two
    // bands' sources, the block-table slice) behind a single wait, then the
    // first copy, then the first two bands; so one HBM round trip precedes
    // the copy instead of a chain of them.
    bf16x8 rreg[DR > 0 ? DR / 16 : 1];  // r of the lane's column: the band's B operand
    BandSrc<DR> pv;                      // sources of the next band
    BandSrc<DR> pv0;                     // (start only) sources of the band before the first
    // WB with whole blocks first: the first bands' sources are requested
    // after the last whole block instead.
    bool band_first = n1 == 0 && ring_phase && rel_active(js_lo);
    if (band_first) {
        load_p(pv0, js_lo - 32);
        load_p(pv, js_lo);
    }
    load_q(C, A.q + trow * DQK, lane);
    auto load_r = [&]() {
#pragma unroll
        for (int st = 0; st < DR / 16; ++st) {
            if (real) {
                rreg[st] = *reinterpret_cast<const bf16x8*>(A.r + trow * DR + 16 * st + 8 * hh);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) rreg[st][i] = (__bf16)0.f;
            }
        }
    };
    // WB with whole blocks first: r is loaded after them, so that it is not
    // held through the blocks that need no bias.
    if (!WB || n1 == 0) load_r();
    init_acc(C);
    // A device length that breaks the caller's contract (fewer keys than new
    // rows, or more keys than the block-table row can address) makes the
    // tile's rows NaN; no table entry past the row is ever read.
    if (ctx < 0 || (long long)L > (long long)A.max_blocks * BS) {
        if (wave_active && real)
            store_out(C, A.out + trow * DV, A.lse ? A.lse + trow : nullptr, true, -INFINITY, INFINITY, lane);
        return;
    }
    bool bad = false;

    int tab_base = kb_lo;
    int tabv = (kb_lo + lane <= kb_hi) ? tab[kb_lo + lane] : -1;
    // first key row (in the K/V caches) of stage s
    auto stage_row = [&](int s, bool& okk) -> size_t {
        const int kb = s / SPB;
        if (kb - tab_base >= 64) {
            tab_base += 64;
            tabv = (tab_base + lane <= kb_hi) ? tab[tab_base + lane] : -1;
        }
        const int phys = __builtin_amdgcn_readlane(tabv, kb - tab_base);
        okk = phys >= 0 && phys < A.num_blocks;
        return okk ? ((size_t)phys * A.Hkv + g) * BS + (size_t)(s % SPB) * HB : 0;
    };

    int koff[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) koff[st] = n * DQK + 8 * ((2 * st + hh) ^ (n & 15));
    int vbo[DV / 32];
    {
        const int gq = lane >> 4, j = lane & 15, vr = 8 * (gq >> 1) + (j >> 2);
#pragma unroll
        for (int dt = 0; dt < DV / 32; ++dt)
            vbo[dt] = vr * DV + 32 * ((dt + vrot<DV>(vr)) & (DV / 32 - 1)) + 16 * (gq & 1) + 4 * (j & 3);
    }

    // T(jb) into the ring. DR > 0: from the rows p, lane (n, hh) holding
    // rows 8 i + 4 hh + 0..3 of column n. DR = 0: the rel pieces as loaded.
    auto band = [&](const BandSrc<DR>& p, int jb) {
        const int par = (jb >> 5) & 1;
        if constexpr (DR > 0) {
            f32x16 Tb = zero16();
#pragma unroll
            for (int st = 0; st < DR / 16; ++st) Tb = mfma32(p.p[st], rreg[st], Tb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = {Tb[4 * i], Tb[4 * i + 1], Tb[4 * i + 2], Tb[4 * i + 3]};
                *reinterpret_cast<f32x4*>(ring + 32 * par + 8 * i + 4 * hh) = v;
            }
            if (par == 0) {
                const f32x4 v = {Tb[0], Tb[1], Tb[2], Tb[3]};
                *reinterpret_cast<f32x4*>(ring + 64 + 4 * hh) = v;
            }
        } else {
            const int q = lane & 7;
            float* dst = ringw + (lane >> 3) * RSTRIDE + 4 * q;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                *reinterpret_cast<f32x4*>(dst + 8 * k * RSTRIDE + 32 * par) = p.p[k];
                if (par == 0 && q < 2) *reinterpret_cast<f32x4*>(dst + 8 * k * RSTRIDE + 64) = p.p[k];
            }
        }
    };
    // bias of subtile js in the score layout (register 8 c + e: key
    // js + 16 c + 8 hh + e)
    auto read_bias = [&](int js, RelVals& rb) {
        const int par = (js >> 5) & 1;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int x = n - 16 * c - 8 * hh + 32 + 32 * par;
            const float* p = ring + ((x - 7) & 63);
#pragma unroll
            for (int e = 0; e < 8; ++e) rb.v[8 * c + e] = p[7 - e];
        }
    };
    auto compute = [&](const __bf16* Kc, const __bf16* Vc, int sub, int js, bool biased) {
        const f32x16 sc = qk_swz(Kc + 32 * sub * DQK, koff, C.qreg);
        RelVals rb;
        if (biased) read_bias(js, rb);
        float x[16];
        sm_logits_rv(C, sc, biased, rb, true, need_mask_of(C, js, A.W), js, A.W, A.R, c1f, l2f, lane, x);
        bf16x8 pb[2];
        float psum;
        if constexpr (WB) {
            // No window: the probabilities against the current reference
            // first. The column max is needed only where a column has no
            // reference yet or some lane's sum says a probability may exceed
            // 2^TAU; the lazy-rescale decision is then the usual one (taken on
            // the max), so the results do not depend on this shortcut. (With a
            // window the first subtiles of a sweep reach the columns at
            // different keys, and computing the max up front measured faster.)
            psum = sm_probs_sum(x, pb);
            if (__any(!C.m_set || psum > PSUM_TRIGGER)) {
                float M = sm_colmax(x);
                if (__any(!C.m_set || sm_trigger(C, M))) {
                    if (__any(!C.m_set)) sm_init_ref(C, M, x);
                    if (__any(sm_trigger(C, M))) sm_rescale(C, M, x);
                    psum = sm_probs_sum(x, pb);
                }
            }
        } else {
            float M = sm_colmax(x);
            if (__any(!C.m_set || sm_trigger(C, M))) {
                if (__any(!C.m_set)) sm_init_ref(C, M, x);
                if (__any(sm_trigger(C, M))) sm_rescale(C, M, x);
            }
            psum = sm_probs_sum(x, pb);
        }
        C.l_sum += psum;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int dt = 0; dt < DV / 32; ++dt)
                C.O[dt] = mfma32(v_operand_rot(Vc + (32 * sub + 16 * c) * DV, vbo[dt], DV), pb[c], C.O[dt]);
        }
    };

    bool ok = false;
    __bf16* const Kw0 = reinterpret_cast<__bf16*>(WBL);  // WB: whole-block buffer 0
    if constexpr (WB) {
        Ks0 = Kw0;
        Vs0 = Ks0 + HB * DQK;
        if constexpr (KV8) {
            Ks1 = Ks0;
            Vs1 = Vs0;
            S8p = reinterpret_cast<uint8_t*>(WBL + WHOLEB);
            ringw = wid < RINGS_IN ? reinterpret_cast<float*>(WBL + HALFB) + wid * RING_W
                                   : reinterpret_cast<float*>(WBL + WHOLEB + S8B) + (wid - RINGS_IN) * RING_W;
        } else {
            Ks1 = Vs0 + HB * DV;
            Vs1 = Ks1 + HB * DQK;
            ringw = reinterpret_cast<float*>(WBL + WHOLEB) + wid * RING_W;
        }
        ring = ringw + n * RSTRIDE;
    }
    if (WB && n1 > 0) {
        const size_t row = stage_row(kb_lo * SPB, ok);
        if constexpr (KV8) {
            if (ok) kv8_dma<DV, 4>(S8p, k8 + row * DQK, v8 + row * DV, wid, lane);
        } else {
            __bf16* K1st = Kw0 + (n1 & 1) * (WHOLEB / 2);  // whole block i goes to buffer (i + n1) mod 2
            if (ok) kv_dma<DV, 4>(K1st, K1st + BS * DQK, A.k + row * DQK, A.v + row * DV, L - kb_lo * BS, wid, lane);
        }
    } else if (ring_phase) {
        const size_t row = stage_row(s_first, ok);
        if constexpr (KV8) {
            if (ok) kv8_dma<DV, NW, HB>(S8p, k8 + row * DQK, v8 + row * DV, wid, lane);
        } else {
            if (ok) kv_dma<DV, NW, HB>(Ks0, Vs0, A.k + row * DQK, A.v + row * DV, L - js_lo, wid, lane);
        }
    }
    int band_js = INT_MIN;  // last band in the ring
    int pv_js = INT_MIN;    // band whose sources pv holds

    // WB: the whole blocks (no row of the tile has bias there). The last one
    // starts the ring phase's first copy into the other buffer; the first two
    // bands' sources are requested after it.
    if constexpr (WB) {
#pragma unroll 1
        for (int i = 0; i < n1; ++i) {
            const int kb = kb_lo + i;
            const __bf16* Kc = KV8 ? Kw0 : Kw0 + ((i + n1) & 1) * (WHOLEB / 2);
            const __bf16* Vc = Kc + BS * DQK;
            __bf16* Kn = Kw0 + ((i + 1 + n1) & 1) * (WHOLEB / 2);
            vm_wait_all();
            lds_barrier();
            const bool ok_cur = ok;
            bad = bad || !ok_cur;
            if constexpr (KV8) {
                kv8_widen<DV>(Kw0, Kw0 + BS * DQK, S8p, L - kb * BS, tid);  // this block, bytes -> bf16
                lds_barrier();                                             // widened block visible, S8 free
                if (i + 1 < n1) {
                    const size_t row = stage_row((kb + 1) * SPB, ok);
                    if (ok) kv8_dma<DV, 4>(S8p, k8 + row * DQK, v8 + row * DV, wid, lane);
                } else if (ring_phase) {
                    const size_t row = stage_row(s_first, ok);
                    if (ok) kv8_dma<DV, NW, HB>(S8p, k8 + row * DQK, v8 + row * DV, wid, lane);
                }
            } else if (i + 1 < n1) {
                const size_t row = stage_row((kb + 1) * SPB, ok);
                if (ok) kv_dma<DV, 4>(Kn, Kn + BS * DQK, A.k + row * DQK, A.v + row * DV, L - (kb + 1) * BS, wid, lane);
            } else if (ring_phase) {
                const size_t row = stage_row(s_first, ok);
                if (ok) kv_dma<DV, NW, HB>(Ks0, Vs0, A.k + row * DQK, A.v + row * DV, L - js_lo, wid, lane);
            }
            if (wave_active && ok_cur) {
#pragma unroll
                for (int sub = 0; sub < 4; ++sub) {
                    const int js = kb * BS + 32 * sub;
                    if (!masked_all(C, js, A.W)) compute(Kc, Vc, sub, js, false);
                }
            }
        }
        if (n1 > 0 && ring_phase) {
            // (requested only now, so that they are not live across the last
            // whole block's compute)
            load_r();
            if (rel_active(js_lo)) {
                load_p(pv0, js_lo - 32);
                load_p(pv, js_lo);
                band_first = true;
            }
            vm_wait_all();
            lds_barrier();  // every wave is done with the buffer that becomes the rings
        }
    }
    if (band_first) {
        band(pv0, js_lo - 32);
        band(pv, js_lo);
        band_js = js_lo;
    }

    // One stage (two subtiles). Each band's sources are requested one subtile
    // ahead; the next stage's first band's at the end of the stage, so they
    // have landed by its barrier.
    auto step = [&](const __bf16* Kc, const __bf16* Vc, __bf16* Kn, __bf16* Vn, int s) {
        vm_wait_all();
        lds_barrier();
        const bool ok_cur = ok;
        bad = bad || !ok_cur;
        const int js0 = s * HB, js1 = js0 + 32;
        if constexpr (KV8) {
            kv8_widen<DV, HB>(Ks0, Vs0, S8p, L - js0, tid);  // this stage, bytes -> bf16
            lds_barrier();                                 // widened stage visible, S8 free
        }
        const bool comp0 = wave_active && ok_cur && !masked_all(C, js0, A.W);
        const bool comp1 = wave_active && ok_cur && !masked_all(C, js1, A.W);
        const bool bias0 = comp0 && bias_on(C, js0, A.R);
        const bool bias1 = comp1 && bias_on(C, js1, A.R);
        if (bias0 && band_js != js0) {
            if (band_js != js0 - 32) {  // the ring lacks the previous band
                load_p(pv, js0 - 32);
                band(pv, js0 - 32);
                pv_js = INT_MIN;
            }
            if (pv_js != js0) load_p(pv, js0);
            band(pv, js0);
            band_js = js0;
        }
        if (s < s_hi) {
            const size_t row = stage_row(s + 1, ok);
            if constexpr (KV8) {
                if (ok) kv8_dma<DV, NW, HB>(S8p, k8 + row * DQK, v8 + row * DV, wid, lane);
            } else {
                if (ok) kv_dma<DV, NW, HB>(Kn, Vn, A.k + row * DQK, A.v + row * DV, L - (s + 1) * HB, wid, lane);
            }
        }
        if (bias1 && band_js == js0) {
            load_p(pv, js1);
            pv_js = js1;
        }
        if (comp0) compute(Kc, Vc, 0, js0, bias0);
        if (bias1) {
            if (band_js != js0) {  // sub 0 had no band: build the ring first
                load_p(pv, js0);
                band(pv, js0);
                pv_js = INT_MIN;
            }
            if (pv_js != js1) load_p(pv, js1);
            band(pv, js1);
            band_js = js1;
        }
        const int jn = js0 + HB;  // the next stage's first subtile
        if (s < s_hi && rel_active(jn)) {
            load_p(pv, jn);
            pv_js = jn;
        }
        if (comp1) compute(Kc, Vc, 1, js1, bias1);
    };
    for (int s = s_first; ring_phase;) {
        step(Ks0, Vs0, Ks1, Vs1, s);
        if (++s > s_hi) break;
        step(Ks1, Vs1, Ks0, Vs0, s);
        if (++s > s_hi) break;
    }

    if (!wave_active || !real) return;
    store_out(C, A.out + trow * DV, A.lse ? A.lse + trow : nullptr, bad, A.sink ? A.sink[trow] : -INFINITY,
              A.gate ? A.gate[trow] : INFINITY, lane, KV8 ? A.v_scale : 1.f);
}

template <int DV, int DR>
__global__ void __launch_bounds__(512) prefill_relproj_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, false, DR>(A);
}

template <int DV, int DR>
__global__ void __launch_bounds__(512) prefill_relproj_logpos_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, true, DR>(A);
}

template <int DV, int DR>
__global__ void __launch_bounds__(512) prefill_relproj_fp8_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, false, DR, true>(A);
}

template <int DV, int DR>
__global__ void __launch_bounds__(512) prefill_relproj_fp8_logpos_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, true, DR, true>(A);
}

// Windowed prefill over a materialised rel, the bias staged through the ring.
template <int DV>
__global__ void __launch_bounds__(512) prefill_ring_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, false, 0>(A);
}

// Prefill without a window: whole blocks, then the ring from the first block with bias.
template <int DV>
__global__ void __launch_bounds__(512) prefill_tail_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, false, 0, false, true>(A);
}

template <int DV>
__global__ void __launch_bounds__(512) prefill_tail_logpos_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, true, 0, false, true>(A);
}

template <int DV>
__global__ void __launch_bounds__(512) prefill_tail_fp8_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, false, 0, true, true>(A);
}

template <int DV>
__global__ void __launch_bounds__(512) prefill_tail_fp8_logpos_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, true, 0, true, true>(A);
}

// The same with the bias made in the kernel.
template <int DV, int DR>
__global__ void __launch_bounds__(512) prefill_relproj_tail_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, false, DR, false, true>(A);
}

template <int DV, int DR>
__global__ void __launch_bounds__(512) prefill_relproj_tail_logpos_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, true, DR, false, true>(A);
}

template <int DV, int DR>
__global__ void __launch_bounds__(512) prefill_relproj_tail_fp8_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, false, DR, true, true>(A);
}

template <int DV, int DR>
__global__ void __launch_bounds__(512) prefill_relproj_tail_fp8_logpos_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, true, DR, true, true>(A);
}

template <int DV>
__global__ void __launch_bounds__(512) prefill_ring_logpos_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, true, 0>(A);
}

template <int DV>
__global__ void __launch_bounds__(512) prefill_ring_fp8_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, false, 0, true>(A);
}

template <int DV>
__global__ void __launch_bounds__(512) prefill_ring_fp8_logpos_kernel(const PrefillArgs A) {
    prefill_ring_body<DV, true, 0, true>(A);
}

// ---------------------------------------------------------------------------
// Split-KV decode
//
// Each of the 4 waves streams subtile w (keys 32 w .. 32 w + 31) of every
// block of its split, independently of the other waves (no barrier in the
// main loop): K goes straight from HBM into the MFMA A-operand registers, V
// into a wave-private LDS tile in natural layout. The split's block-table
// slice is held in one register (lane i = entry i) and read with readlane, so
// no block waits on a dependent table load. The four waves' partial softmax
// states are merged through LDS at the end.
// ---------------------------------------------------------------------------
template <int DV, int NW = 4>
struct DecodeLds {
    static constexpr int V_BYTES = 32 * vrow<DV>() * 2;
    static constexpr int R_BYTES = 32 * RROW * 4;
    static constexpr int WAVE = V_BYTES + R_BYTES;
    static constexpr int MERGE = NW * 32 * DV * 4 + 2 * NW * 32 * 4;
    static constexpr int TOTAL = (NW * WAVE > MERGE) ? NW * WAVE : MERGE;
};

// K subtile (32 keys) of one block, in the MFMA A-operand layout: lane holds
// key 32 sub + perm32(lane & 31), dims 16 st + 8 (lane >> 5) .. +8.
__device__ __forceinline__ void load_k_sub(bf16x8 (&kr)[8], const uint16_t* kblk, int sub, int lane) {
    const uint16_t* row = kblk + (32 * sub + perm32(lane & 31)) * DQK + 8 * (lane >> 5);
#pragma unroll
    for (int st = 0; st < 8; ++st) kr[st] = *reinterpret_cast<const bf16x8*>(row + 16 * st);
}

// V subtile (32 keys x DV) as 16-byte pieces, lane takes pieces lane + 64 k;
// keys at or past `nvalid` (beyond the sequence) are zeros.
template <int DV>
struct VSub {
    static constexpr int PIECES = 32 * (DV / 8) / 64;  // per lane
    u32x4 r[PIECES];
};

template <int DV>
__device__ __forceinline__ void load_v_sub(VSub<DV>& v, const uint16_t* vblk, int sub, int nvalid, int lane) {
#pragma unroll
    for (int k = 0; k < VSub<DV>::PIECES; ++k) {
        const int p = lane + 64 * k;
        const int key = 32 * sub + p / (DV / 8), c = p % (DV / 8);
        v.r[k] = key < nvalid ? *reinterpret_cast<const u32x4*>(vblk + key * DV + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }
}

template <int DV>
__device__ __forceinline__ void store_v_sub(__bf16* Vw, const VSub<DV>& v, int lane) {
#pragma unroll
    for (int k = 0; k < VSub<DV>::PIECES; ++k) {
        const int p = lane + 64 * k;
        *reinterpret_cast<u32x4*>(Vw + (p / (DV / 8)) * vrow<DV>() + 8 * (p % (DV / 8))) = v.r[k];
    }
}

// load_k_sub for e4m3 K, with the head dimension taken in another order (the
// same for q, see load_q8) so that one 16-byte load feeds two score MFMAs:
// step st of lane half hh covers dims 32 (st >> 1) + 16 hh + 8 (st & 1) .. +8.
__device__ __forceinline__ void load_k_sub8(u32x2 (&kr)[8], const uint8_t* kblk, int sub, int lane) {
    const uint8_t* row = kblk + (32 * sub + perm32(lane & 31)) * DQK + 16 * (lane >> 5);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(row + 32 * s2);
        kr[2 * s2] = u32x2{w[0], w[1]};
        kr[2 * s2 + 1] = u32x2{w[2], w[3]};
    }
}

// V subtile of e4m3 V as 16-byte pieces of 16 values; widened to bf16 when
// stored to LDS (same LDS layout as store_v_sub).
template <int DV>
struct VSub8 {
    static constexpr int PIECES = 32 * (DV / 16) / 64;  // per lane
    u32x4 r[PIECES];
};

template <int DV>
__device__ __forceinline__ void load_v_sub8(VSub8<DV>& v, const uint8_t* vblk, int sub, int nvalid, int lane) {
#pragma unroll
    for (int k = 0; k < VSub8<DV>::PIECES; ++k) {
        const int p = lane + 64 * k;
        const int key = 32 * sub + p / (DV / 16), c = p % (DV / 16);
        v.r[k] = key < nvalid ? *reinterpret_cast<const u32x4*>(vblk + key * DV + 16 * c) : u32x4{0u, 0u, 0u, 0u};
    }
}

template <int DV>
__device__ __forceinline__ void store_v_sub8(__bf16* Vw, const VSub8<DV>& v, int lane) {
#pragma unroll
    for (int k = 0; k < VSub8<DV>::PIECES; ++k) {
        const int p = lane + 64 * k;
        __bf16* dst = Vw + (p / (DV / 16)) * vrow<DV>() + 16 * (p % (DV / 16));
        const u32x4 w = v.r[k];
        *reinterpret_cast<bf16x8*>(dst) = fp8x8_to_bf16(u32x2{w[0], w[1]});
        *reinterpret_cast<bf16x8*>(dst + 8) = fp8x8_to_bf16(u32x2{w[2], w[3]});
    }
}

// K/V element type of the decode kernels: bf16 (KV8 = false) or e4m3.
template <bool KV8>
struct Kv {
    typedef bf16x8 KReg;
    template <int DV>
    using VRegs = VSub<DV>;
    static constexpr int ESZ = 2;
    __device__ static bf16x8 op(const KReg& k) { return k; }
    __device__ static void k_sub(KReg (&kr)[8], const char* kblk, int sub, int lane) {
        load_k_sub(kr, reinterpret_cast<const uint16_t*>(kblk), sub, lane);
    }
    template <int DV>
    __device__ static void v_load(VRegs<DV>& v, const char* vblk, int sub, int nvalid, int lane) {
        load_v_sub<DV>(v, reinterpret_cast<const uint16_t*>(vblk), sub, nvalid, lane);
    }
    template <int DV>
    __device__ static void v_store(__bf16* Vw, const VRegs<DV>& v, int lane) {
        store_v_sub<DV>(Vw, v, lane);
    }
};

template <>
struct Kv<true> {
    typedef u32x2 KReg;
    template <int DV>
    using VRegs = VSub8<DV>;
    static constexpr int ESZ = 1;
    __device__ static bf16x8 op(const KReg& k) { return fp8x8_to_bf16(k); }
    __device__ static void k_sub(KReg (&kr)[8], const char* kblk, int sub, int lane) {
        load_k_sub8(kr, reinterpret_cast<const uint8_t*>(kblk), sub, lane);
    }
    template <int DV>
    __device__ static void v_load(VRegs<DV>& v, const char* vblk, int sub, int nvalid, int lane) {
        load_v_sub8<DV>(v, reinterpret_cast<const uint8_t*>(vblk), sub, nvalid, lane);
    }
    template <int DV>
    __device__ static void v_store(__bf16* Vw, const VRegs<DV>& v, int lane) {
        store_v_sub8<DV>(Vw, v, lane);
    }
};

// NW = 4: wave w takes the 32-key subtile w of every block of the split.
// NW = 8 (one workgroup per CU): waves 4..7 take the odd blocks and waves
// 0..3 the even ones, so a workgroup keeps two blocks of loads in flight.
template <int DV, bool KV8, bool LS, int NW = 4>
__device__ __forceinline__ void decode_split_body(const DecodeArgs A) {
    using KV = Kv<KV8>;
    using Lds = DecodeLds<DV, NW>;
    const char* const kbase = reinterpret_cast<const char*>(A.k);
    const char* const vbase = reinterpret_cast<const char*>(A.v);
    __shared__ __attribute__((aligned(16))) char smem[Lds::TOTAL];

    const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 31, hh = lane >> 5;
    constexpr int STEP = NW / 4;                       // blocks between a wave's steps
    const int sub = wid & 3, par = wid >> 2;            // subtile in the block; block parity
    int id = blockIdx.x;
    const int g = id % A.Hkv;
    id /= A.Hkv;
    const int b = id % A.batch;
    id /= A.batch;
    const int cg = id % A.n_cg;
    const int split = id / A.n_cg;

    // With no window a split's first block does not depend on the sequence
    // length, so its block-table slice is requested before that arrives.
    const int tab_spec_lo = split * A.bps + par;
    const int* const tab_row = A.tables + (long long)b * A.max_blocks;
    const int tab_spec = (A.W == 0 && tab_spec_lo + lane < A.max_blocks) ? tab_row[tab_spec_lo + lane] : -1;
    const int L = A.seq_lens[b];
    const int ncols = A.G * A.n_q;
    const int c = cg * 32 + n;
    const bool real = c < ncols;
    const int tt = real ? c / A.G : 0;
    const int hl = real ? c % A.G : 0;
    const int h = g * A.G + hl;
    const long long trow = (long long)(b * A.n_q + tt) * A.Hq + h;
    const float fls = (LS && real) ? A.lscale[b * A.n_q + tt] : 1.f;  // the row's logit scale
    const float c1f = A.c1 * fls, l2f = LOG2E * fls;

    Cols<DV> C;
    C.pos = real ? L - A.n_q + tt : -1;
    C.relrow = A.rel + trow * A.R;
    const int c_hi = min(cg * 32 + 31, ncols - 1);
    C.w_lo = L - A.n_q + (cg * 32) / A.G;
    C.w_hi = L - A.n_q + c_hi / A.G;
    C.phantom = c_hi < cg * 32 + 31;
    if constexpr (KV8)
        load_q8(C, A.q + trow * DQK, lane);
    else
        load_q(C, A.q + trow * DQK, lane);
    init_acc(C);

    const int nb = L / BS + (L % BS != 0);
    const int kb_first = A.W > 0 ? max(0, (L - A.n_q) - A.W + 1) / BS : 0;
    const int s_lo = kb_first + split * A.bps;
    // A device length that breaks the caller's contract (fewer keys than
    // query tokens, more than the block-table row addresses, or more than the
    // split plan made from the host's max_seq_len covers) gives NaN rows; no
    // table entry past the row is read.
    const bool len_bad = L < A.n_q || nb > A.max_blocks || nb > kb_first + A.splits * A.bps;
    const int s_hi = len_bad ? s_lo : min(s_lo + A.bps, nb);
    __bf16* Vw = reinterpret_cast<__bf16*>(smem + wid * Lds::WAVE);
    float* Rw = reinterpret_cast<float*>(smem + wid * Lds::WAVE + Lds::V_BYTES);
    const int* tab = tab_row;
    bool bad = len_bad;

    // This wave's subtiles that are not entirely masked form one run of
    // blocks ka, ka + STEP, ..., kz.
    int ka = s_lo + par, kz = ka <= s_hi - 1 ? ka + (s_hi - 1 - ka) / STEP * STEP : ka - STEP;
    while (ka <= kz && masked_all(C, ka * BS + 32 * sub, A.W)) ka += STEP;
    while (kz >= ka && masked_all(C, kz * BS + 32 * sub, A.W)) kz -= STEP;

    // split's block-table slice, lane i = entry tab_base + i
    int tab_base = ka;
    int tabv = (ka + lane <= kz) ? (A.W == 0 && ka == tab_spec_lo ? tab_spec : tab[ka + lane]) : -1;
    auto phys_of = [&](int kb) {
        if (kb - tab_base >= 64) {
            tab_base += 64;
            tabv = (tab_base + lane <= kz) ? tab[tab_base + lane] : -1;
        }
        return __builtin_amdgcn_readlane(tabv, kb - tab_base);
    };

    if constexpr (DV <= 64) {
        // the dv 64 accumulators leave room for the next block's K operands
        // and V subtile: each wave keeps two blocks of loads in flight
        auto block_base = [&](int kb, bool& okk) -> size_t {
            const int phys = phys_of(kb);
            okk = phys >= 0 && phys < A.num_blocks;
            return okk ? ((size_t)phys * A.Hkv + g) * BS : 0;
        };
        typename KV::KReg kr[8];
        typename KV::template VRegs<DV> vs;
        // the bias of a subtile is loaded one block ahead too, so that the
        // blocks near the queries do not wait a memory round trip each (the
        // per-row scales of the log-position variant leave no registers for
        // it: there it is loaded in the block's own step)
        constexpr bool REL_AHEAD = !LS;
        RelRegs rr;
        bool ok_cur = false;
        if (ka <= kz) {
            const size_t base = block_base(ka, ok_cur);
            if (ok_cur) {
                KV::k_sub(kr, kbase + base * DQK * KV::ESZ, sub, lane);
                KV::template v_load<DV>(vs, vbase + base * DV * KV::ESZ, sub, L - ka * BS, lane);
            }
            if (REL_AHEAD && bias_on(C, ka * BS + 32 * sub, A.R))
                rel_load(rr, C.relrow, C.pos, ka * BS + 32 * sub, A.R, lane);
        }
#pragma unroll 1
        for (int kb = ka; kb <= kz; kb += STEP) {
            const int js = kb * BS + 32 * sub;
            bool ok_next = false;
            const size_t base_next = kb < kz ? block_base(kb + STEP, ok_next) : 0;
            const bool brel = bias_on(C, js, A.R);
            const bool brel_next = kb < kz && bias_on(C, js + STEP * BS, A.R);
            if (!ok_cur) {
                bad = true;
                if (ok_next) {
                    KV::k_sub(kr, kbase + base_next * DQK * KV::ESZ, sub, lane);
                    KV::template v_load<DV>(vs, vbase + base_next * DV * KV::ESZ, sub, L - (kb + STEP) * BS, lane);
                }
                if (REL_AHEAD && brel_next) rel_load(rr, C.relrow, C.pos, js + STEP * BS, A.R, lane);
                ok_cur = ok_next;
                continue;
            }
            if (!REL_AHEAD && brel) rel_load(rr, C.relrow, C.pos, js, A.R, lane);
            KV::template v_store<DV>(Vw, vs, lane);
            if (ok_next) KV::template v_load<DV>(vs, vbase + base_next * DV * KV::ESZ, sub, L - (kb + STEP) * BS, lane);
            bf16x8 kb16[8];
#pragma unroll
            for (int st = 0; st < 8; ++st) kb16[st] = KV::op(kr[st]);
            const f32x16 s = qk_regs(kb16, C.qreg);
            if (ok_next) KV::k_sub(kr, kbase + base_next * DQK * KV::ESZ, sub, lane);
            if (brel) rel_store(Rw, rr, lane);
            if (REL_AHEAD && brel_next) rel_load(rr, C.relrow, C.pos, js + STEP * BS, A.R, lane);
            __builtin_amdgcn_wave_barrier();
            softmax_pv<DV>(C, s, brel, rel_row_ptr(Rw, C.pos, lane), js, A.W, c1f, l2f, lane,
                           [&](int dt, int cc) { return v_operand(Vw, vrow<DV>(), 16 * cc, 32 * dt, lane); });
            __builtin_amdgcn_wave_barrier();
            ok_cur = ok_next;
        }
    } else {
        for (int kb = ka; kb <= kz; kb += STEP) {
            const int js = kb * BS + 32 * sub;
            const int phys = phys_of(kb);
            if (phys < 0 || phys >= A.num_blocks) {
                bad = true;
                continue;
            }
            const size_t base = ((size_t)phys * A.Hkv + g) * BS;
            const bool brel = bias_on(C, js, A.R);
            typename KV::KReg kr[8];
            typename KV::template VRegs<DV> vs;
            KV::k_sub(kr, kbase + base * DQK * KV::ESZ, sub, lane);
            KV::template v_load<DV>(vs, vbase + base * DV * KV::ESZ, sub, L - kb * BS, lane);
            KV::template v_store<DV>(Vw, vs, lane);
            RelRegs rr;
            if (brel) rel_load(rr, C.relrow, C.pos, js, A.R, lane);
            bf16x8 kb16[8];
#pragma unroll
            for (int st = 0; st < 8; ++st) kb16[st] = KV::op(kr[st]);
            const f32x16 s = qk_regs(kb16, C.qreg);
            if (brel) rel_store(Rw, rr, lane);
            __builtin_amdgcn_wave_barrier();
            softmax_pv<DV>(C, s, brel, rel_row_ptr(Rw, C.pos, lane), js, A.W, c1f, l2f, lane,
                           [&](int dt, int cc) { return v_operand(Vw, vrow<DV>(), 16 * cc, 32 * dt, lane); });
            __builtin_amdgcn_wave_barrier();
        }
    }

    // Merge the waves' partial states through LDS.
    __syncthreads();
    float* Om = reinterpret_cast<float*>(smem);   // [NW][32][DV]
    float* Mm = Om + NW * 32 * DV;                // [NW][32] reference max (or -inf)
    float* Lm = Mm + NW * 32;                     // [NW][32] row sums
    const float l_tot = C.l_sum + xor32(C.l_sum);
    const bool any_bad = __syncthreads_or(bad);
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = C.O[dt][4 * q4 + k];
            *reinterpret_cast<f32x4*>(Om + (wid * 32 + n) * DV + 32 * dt + 8 * q4 + 4 * hh) = o;
        }
    }
    if (hh == 0) {
        Mm[wid * 32 + n] = C.m_set ? C.m_ref : -INFINITY;
        Lm[wid * 32 + n] = l_tot;
    }
    __syncthreads();

    for (int e = tid; e < 32 * DV; e += 64 * NW) {
        const int col = e / DV, dv = e % DV;
        const int cc = cg * 32 + col;
        if (cc >= ncols) continue;
        float mw[NW], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            mw[w] = Mm[w * 32 + col];
            M = fmaxf(M, mw[w]);
        }
        float den = 0.f, num = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = __builtin_amdgcn_exp2f(mw[w] - M);  // exp2(-inf) = 0
                den += f * Lm[w * 32 + col];
                num += f * Om[(w * 32 + col) * DV + dv];
            }
        }
        const int ctt = cc / A.G, chl = cc % A.G;
        const long long prow = ((long long)(b * A.n_q + ctt) * A.Hq + (g * A.G + chl)) * A.splits + split;
        A.part_o[prow * DV + dv] = any_bad ? NAN : (M > -INFINITY ? num / den * A.v_scale : 0.f);
        if (dv == 0) {
            A.part_lse[prow] = any_bad ? NAN : (M > -INFINITY ? (M + __log2f(den)) * LN2 : -INFINITY);
        }
    }
}

template <int DV, bool KV8>
__global__ void __launch_bounds__(256, 2) decode_split_kernel(const DecodeArgs A) {
    decode_split_body<DV, KV8, false>(A);
}

template <int DV, bool KV8>
__global__ void __launch_bounds__(512) decode_split8_kernel(const DecodeArgs A) {
    decode_split_body<DV, KV8, false, 8>(A);
}

template <int DV, bool KV8>
__global__ void __launch_bounds__(256, 2) decode_split_logpos_kernel(const DecodeArgs A) {
    decode_split_body<DV, KV8, true>(A);
}

template <int DV, bool KV8>
__global__ void __launch_bounds__(512) decode_split8_logpos_kernel(const DecodeArgs A) {
    decode_split_body<DV, KV8, true, 8>(A);
}

// ---------------------------------------------------------------------------
// Decode for 33 to 64 columns (G * n_q), bf16 K/V: one workgroup of 8 waves
// per (sequence, KV head, split) covers both 32-column groups. Waves 0-3
// take group 0 and waves 4-7 group 1, wave w subtile w & 3 of every block, so
// the two waves of a subtile share its K/V: each 128-key block is copied from
// HBM into LDS once (global_load_lds into double buffers, in the prefill's
// swizzled-K / rotated-V layouts, all 8 waves issuing the copies) and both
// groups read it there, instead of each group's workgroup loading every
// block into its own registers. The next block's copy overlaps the current
// block's compute; the bias of the next block's subtile is requested during
// the current one. Scores, softmax and P.V are the prefill's. The partial
// state of each group is merged over its 4 waves through LDS, as in the other
// decode kernels.
// ---------------------------------------------------------------------------
template <int DV>
struct PairLds {
    static constexpr int KV_BYTES = 2 * BS * DQK * 2 + 2 * BS * DV * 2;   // K0, K1, V0, V1
    static constexpr int MERGE = 8 * 32 * DV * 4 + 2 * 8 * 32 * 4;
    static constexpr int TOTAL = KV_BYTES > MERGE ? KV_BYTES : MERGE;
};

template <int DV, bool LS>
__device__ __forceinline__ void decode_pair_body(const DecodeArgs A) {
    __shared__ __attribute__((aligned(16))) char smem[PairLds<DV>::TOTAL];
    __bf16* const K0 = reinterpret_cast<__bf16*>(smem);
    __bf16* const K1 = K0 + BS * DQK;
    __bf16* const V0 = K1 + BS * DQK;
    __bf16* const V1 = V0 + BS * DV;

    const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 31,
              hh = lane >> 5;
    const int grp = wid >> 2, sub = wid & 3;
    int id = blockIdx.x;
    const int g = id % A.Hkv;
    id /= A.Hkv;
    const int b = id % A.batch;
    const int split = id / A.batch;

    const int L = A.seq_lens[b];
    const int ncols = A.G * A.n_q;   // 33 .. 64
    const int c = grp * 32 + n;
    const bool real = c < ncols;
    const int tt = real ? c / A.G : 0;
    const int hl = real ? c % A.G : 0;
    const int h = g * A.G + hl;
    const long long trow = (long long)(b * A.n_q + tt) * A.Hq + h;
    const float fls = (LS && real) ? A.lscale[b * A.n_q + tt] : 1.f;  // the row's logit scale
    const float c1f = A.c1 * fls, l2f = LOG2E * fls;

    Cols<DV> C;
    C.pos = real ? L - A.n_q + tt : -1;
    C.relrow = A.rel + trow * A.R;
    const int c_hi = min(grp * 32 + 31, ncols - 1);
    C.w_lo = L - A.n_q + (grp * 32) / A.G;
    C.w_hi = L - A.n_q + c_hi / A.G;
    C.phantom = c_hi < grp * 32 + 31;
    load_q(C, A.q + trow * DQK, lane);
    init_acc(C);

    const int nb = L / BS + (L % BS != 0);
    const int kb_first = A.W > 0 ? max(0, (L - A.n_q) - A.W + 1) / BS : 0;
    const int s_lo = kb_first + split * A.bps;
    // a device length outside the caller's contract gives NaN rows (as the
    // other decode kernels); no table entry past the row is read
    const bool len_bad = L < A.n_q || nb > A.max_blocks || nb > kb_first + A.splits * A.bps;
    const int s_hi = len_bad ? s_lo : min(s_lo + A.bps, nb);
    const int ka = s_lo, kz = s_hi - 1;
    bool bad = len_bad;

    const int* const tab = A.tables + (long long)b * A.max_blocks;
    int tab_base = ka;
    int tabv = (ka + lane <= kz) ? tab[ka + lane] : -1;
    auto block_base = [&](int kb, bool& okk) -> size_t {
        if (kb - tab_base >= 64) {
            tab_base += 64;
            tabv = (tab_base + lane <= kz) ? tab[tab_base + lane] : -1;
        }
        const int phys = __builtin_amdgcn_readlane(tabv, kb - tab_base);
        okk = phys >= 0 && phys < A.num_blocks;
        return okk ? ((size_t)phys * A.Hkv + g) * BS : 0;
    };
    auto rel_active = [&](int js) { return !masked_all(C, js, A.W) && bias_on(C, js, A.R); };
    auto rel_inside = [&](int js) { return !C.phantom && C.w_lo - js - 31 >= 0 && C.w_hi - js < A.R; };

    int koff[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) koff[st] = n * DQK + 8 * ((2 * st + hh) ^ (n & 15));
    int vbo[DV / 32];
    {
        const int gq = lane >> 4, j = lane & 15, vr = 8 * (gq >> 1) + (j >> 2);
#pragma unroll
        for (int dt = 0; dt < DV / 32; ++dt)
            vbo[dt] = vr * DV + 32 * ((dt + vrot<DV>(vr)) & (DV / 32 - 1)) + 16 * (gq & 1) + 4 * (j & 3);
    }

    bool ok = false;
    RelVals rv[2];  // bias of this block's subtile and of the next block's
    if (ka <= kz) {
        const size_t base = block_base(ka, ok);
        if (ok) kv_dma<DV, 8>(K0, V0, A.k + base * DQK, A.v + base * DV, L - ka * BS, wid, lane);
        if (rel_active(ka * BS + 32 * sub))
            rel_fetch(rv[0], C.relrow, C.pos, ka * BS + 32 * sub, A.R, rel_inside(ka * BS + 32 * sub), lane);
    }

    auto step = [&](const __bf16* Kc, const __bf16* Vc, __bf16* Kn, __bf16* Vn, int kb, const RelVals& rcur,
                    RelVals& rnext) {
        vm_wait_all();
        lds_barrier();  // this block's copy is in; every wave is done with the other buffers
        const bool ok_cur = ok;
        bad = bad || !ok_cur;
        if (kb < kz) {
            const size_t base = block_base(kb + 1, ok);
            if (ok) kv_dma<DV, 8>(Kn, Vn, A.k + base * DQK, A.v + base * DV, L - (kb + 1) * BS, wid, lane);
        }
        const int js = kb * BS + 32 * sub;
        const bool computed = ok_cur && !masked_all(C, js, A.W);
        float x[16];
        float M = -INFINITY;
        if (computed) {
            const f32x16 sc = qk_swz(Kc + 32 * sub * DQK, koff, C.qreg);
            M = sm_scores_rv(C, sc, rel_active(js), rcur, rel_inside(js), need_mask_of(C, js, A.W), js, A.W, A.R,
                             c1f, l2f, lane, x);
        }
        const int jn = js + BS;  // this wave's subtile of the next block
        if (kb < kz && rel_active(jn)) rel_fetch(rnext, C.relrow, C.pos, jn, A.R, rel_inside(jn), lane);
        if (computed) {
            if (__any(!C.m_set || sm_trigger(C, M))) {
                if (__any(!C.m_set)) sm_init_ref(C, M, x);
                if (__any(sm_trigger(C, M))) sm_rescale(C, M, x);
            }
            bf16x8 pb[2];
            sm_probs(C, x, pb);
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
                for (int dt = 0; dt < DV / 32; ++dt)
                    C.O[dt] = mfma32(v_operand_rot(Vc + (32 * sub + 16 * cc) * DV, vbo[dt], DV), pb[cc], C.O[dt]);
            }
        }
    };
    for (int kb = ka; kb <= kz;) {
        step(K0, V0, K1, V1, kb, rv[0], rv[1]);
        if (kb == kz) break;
        ++kb;
        step(K1, V1, K0, V0, kb, rv[1], rv[0]);
        if (kb == kz) break;
        ++kb;
    }

    // Merge each group's 4 partial states through LDS (the K/V buffers are
    // free once every wave has passed the barrier).
    __syncthreads();
    float* Om = reinterpret_cast<float*>(smem);   // [8][32][DV]
    float* Mm = Om + 8 * 32 * DV;                 // [8][32] reference max (or -inf)
    float* Lm = Mm + 8 * 32;                      // [8][32] row sums
    const float l_tot = C.l_sum + xor32(C.l_sum);
    const bool any_bad = __syncthreads_or(bad);
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = C.O[dt][4 * q4 + k];
            *reinterpret_cast<f32x4*>(Om + (wid * 32 + n) * DV + 32 * dt + 8 * q4 + 4 * hh) = o;
        }
    }
    // a column that saw any key has l_tot >= 1 (its reference's own term);
    // one that saw none has l_tot = 0 (its reference was never set)
    if (hh == 0) {
        Mm[wid * 32 + n] = l_tot > 0.f ? C.m_ref : -INFINITY;
        Lm[wid * 32 + n] = l_tot;
    }
    __syncthreads();

    for (int e = tid; e < 64 * DV; e += 512) {
        const int col = e / DV, dv = e % DV;  // column 0 .. 63 = group * 32 + lane column
        if (col >= ncols) continue;
        const int w0 = 4 * (col >> 5), cn = col & 31;
        float mw[4], Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = Mm[(w0 + w) * 32 + cn];
            Mx = fmaxf(Mx, mw[w]);
        }
        float den = 0.f, num = 0.f;
        if (Mx > -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = __builtin_amdgcn_exp2f(mw[w] - Mx);  // exp2(-inf) = 0
                den += f * Lm[(w0 + w) * 32 + cn];
                num += f * Om[((w0 + w) * 32 + cn) * DV + dv];
            }
        }
        const int ctt = col / A.G, chl = col % A.G;
        const long long prow = ((long long)(b * A.n_q + ctt) * A.Hq + (g * A.G + chl)) * A.splits + split;
        A.part_o[prow * DV + dv] = any_bad ? NAN : (Mx > -INFINITY ? num / den : 0.f);
        if (dv == 0) A.part_lse[prow] = any_bad ? NAN : (Mx > -INFINITY ? (Mx + __log2f(den)) * LN2 : -INFINITY);
    }
}

template <int DV>
__global__ void __launch_bounds__(512) decode_pair_kernel(const DecodeArgs A) {
    decode_pair_body<DV, false>(A);
}

template <int DV>
__global__ void __launch_bounds__(512) decode_pair_logpos_kernel(const DecodeArgs A) {
    decode_pair_body<DV, true>(A);
}

// ---------------------------------------------------------------------------
// Split-KV decode, 16-column variant (G * n_q <= 16, e.g. one token of 4
// query heads per KV head). Same work split as decode_split_kernel, but the
// scores use v_mfma_f32_16x16x32_bf16 with 16 (head, token) columns per wave,
// which halves the query, score and accumulator registers; the room goes to a
// prefetch of the next block's K operands and V subtile, so every wave keeps
// two blocks of loads in flight.
//
// Layouts (lane l, column c = l & 15, lane group q = l >> 4):
//   S^T half h (16 keys x 16 columns): MFMA row m holds key 8 (m/4) + 4 h +
//   m%4, so lane l gets keys 8 q + 4 h + j (j = 0..3): the lane's 8 keys of
//   the 32-key subtile are 8 q .. 8 q + 7, exactly the B operand of P.V.
//   O^T tile t (16 dims x 16 columns): lane holds dims 16 t + 4 q + j.
// ---------------------------------------------------------------------------
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mfma16(const bf16x8& a, const bf16x8& b, const f32x4v& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one column's 4 groups)
__device__ __forceinline__ float groups_max(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t a = r[0], b = r[1];
    return halves_max(fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
}

__device__ __forceinline__ float groups_sum(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t a = r[0], b = r[1];
    const float s = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
    const uint32_t w = __builtin_bit_cast(uint32_t, s);
    const auto r2 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    const uint32_t c = r2[0], d = r2[1];
    return __builtin_bit_cast(float, c) + __builtin_bit_cast(float, d);
}

// K operands of one 32-key subtile: kr[2 h + ... ] in order (h, s):
// lane loads key 32 sub + 8 (m/4) + 4 h + m%4 (m = l & 15), dims 32 s + 8 q.
// e4m3 K: the head dimension is taken in a different order (the same for q,
// see dims16_e4m3) so that each 16-byte load feeds two score MFMAs: step st
// of lane group q covers dims 16 (q + 4 (st >> 1)) + 8 (st & 1) + 0..7.
__device__ __forceinline__ int dims16_e4m3(int st, int q) { return 16 * (q + 4 * (st >> 1)) + 8 * (st & 1); }

__device__ __forceinline__ void load_k16(u32x2 (&kr)[8], const uint8_t* kblk, int sub, int lane) {
    const int m = lane & 15, q = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint8_t* row = kblk + (32 * sub + 8 * (m >> 2) + 4 * h + (m & 3)) * DQK;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(row + dims16_e4m3(2 * s2, q));
            kr[4 * h + 2 * s2] = u32x2{w[0], w[1]};
            kr[4 * h + 2 * s2 + 1] = u32x2{w[2], w[3]};
        }
    }
}

__device__ __forceinline__ void load_k16(bf16x8 (&kr)[8], const uint16_t* kblk, int sub, int lane) {
    const int m = lane & 15, q = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint16_t* row = kblk + (32 * sub + 8 * (m >> 2) + 4 * h + (m & 3)) * DQK + 8 * q;
#pragma unroll
        for (int st = 0; st < 4; ++st) kr[4 * h + st] = *reinterpret_cast<const bf16x8*>(row + 32 * st);
    }
}

// P.V A operand for dim tile t from V in natural layout (row stride vs):
// lane gets V[8 q + 0..7][16 t + (l & 15)] via two transposed reads (lane j
// of a 16-lane group takes element j%4 from the address of lane 4k + j/4).
__device__ __forceinline__ bf16x8 v16_operand(const __bf16* Vs, int vs, int t, int lane) {
    const int q = lane >> 4, j = lane & 15;
    const __bf16* p = Vs + (8 * q + (j >> 2)) * vs + 16 * t + 4 * (j & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * vs));
    union {
        s16x4 h[2];
        bf16x8 v;
    } u;
    u.h[0] = lo;
    u.h[1] = hi;
    return u.v;
}

template <int DV>
struct Decode16Lds {
    static constexpr int V_BYTES = 32 * vrow<DV>() * 2;
    static constexpr int MERGE = 4 * 16 * DV * 4 + 2 * 4 * 16 * 4;
    static constexpr int TOTAL = (4 * V_BYTES > MERGE) ? 4 * V_BYTES : MERGE;
};

template <int DV, bool KV8, bool LS>
__device__ __forceinline__ void decode16_split_body(const DecodeArgs A) {
    using KV = Kv<KV8>;
    typedef typename std::conditional<KV8, uint8_t, uint16_t>::type KElem;
    const KElem* const kel = reinterpret_cast<const KElem*>(A.k);
    const KElem* const vel = reinterpret_cast<const KElem*>(A.v);
    __shared__ __attribute__((aligned(16))) char smem[Decode16Lds<DV>::TOTAL];

    const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, q = lane >> 4;
    int id = blockIdx.x;
    const int g = id % A.Hkv;
    id /= A.Hkv;
    const int b = id % A.batch;
    id /= A.batch;
    const int split = id / A.n_cg;  // n_cg == 1 for this variant

    // With no window a split's first block does not depend on the sequence
    // length, so its block-table slice is requested before that arrives.
    const int tab_spec_lo = split * A.bps;
    const int* const tab_row = A.tables + (long long)b * A.max_blocks;
    const int tab_spec = (A.W == 0 && tab_spec_lo + lane < A.max_blocks) ? tab_row[tab_spec_lo + lane] : -1;
    const int L = A.seq_lens[b];
    const int ncols = A.G * A.n_q;
    const bool real = c < ncols;
    const int tt = real ? c / A.G : 0;
    const int h = g * A.G + (real ? c % A.G : 0);
    const long long trow = (long long)(b * A.n_q + tt) * A.Hq + h;
    const int pos = real ? L - A.n_q + tt : -1;
    const float* relrow = A.rel + trow * A.R;
    const float fls = (LS && real) ? A.lscale[b * A.n_q + tt] : 1.f;  // the row's logit scale
    const float c1f = A.c1 * fls, l2f = LOG2E * fls;
    // wave-uniform column range (positions of the first and last real column)
    const int w_lo = L - A.n_q, w_hi = L - A.n_q + (ncols - 1) / A.G;
    const bool phantom = ncols < 16;

    bf16x8 qreg[4];
    // as load_q: a column past the last real one reads a real row (over
    // e4m3 K/V in the dimension order of load_k16)
#pragma unroll
    for (int st = 0; st < 4; ++st)
        qreg[st] = *reinterpret_cast<const bf16x8*>(A.q + trow * DQK + (KV8 ? dims16_e4m3(st, q) : 32 * st + 8 * q));
    f32x4v O[DV / 16];
#pragma unroll
    for (int t = 0; t < DV / 16; ++t) O[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
    float m_ref = 0.f, l_sum = 0.f;
    bool m_set = false;

    const int nb = L / BS + (L % BS != 0);
    const int kb_first = A.W > 0 ? max(0, (L - A.n_q) - A.W + 1) / BS : 0;
    const int s_lo = kb_first + split * A.bps;
    // A device length that breaks the caller's contract (fewer keys than
    // query tokens, more than the block-table row addresses, or more than the
    // split plan made from the host's max_seq_len covers) gives NaN rows; no
    // table entry past the row is read.
    const bool len_bad = L < A.n_q || nb > A.max_blocks || nb > kb_first + A.splits * A.bps;
    const int s_hi = len_bad ? s_lo : min(s_lo + A.bps, nb);
    __bf16* Vw = reinterpret_cast<__bf16*>(smem + wid * Decode16Lds<DV>::V_BYTES);
    const int* tab = tab_row;
    bool bad = len_bad;

    auto masked_all16 = [&](int js) { return js > w_hi || (A.W > 0 && w_lo - (js + 31) >= A.W); };
    int ka = s_lo, kz = s_hi - 1;
    while (ka <= kz && masked_all16(ka * BS + 32 * wid)) ++ka;
    while (kz >= ka && masked_all16(kz * BS + 32 * wid)) --kz;

    int tab_base = ka;
    int tabv = (ka + lane <= kz) ? (A.W == 0 && ka == tab_spec_lo ? tab_spec : tab[ka + lane]) : -1;
    auto block_base = [&](int kb, bool& okk) -> size_t {
        if (kb - tab_base >= 64) {
            tab_base += 64;
            tabv = (tab_base + lane <= kz) ? tab[tab_base + lane] : -1;
        }
        const int phys = __builtin_amdgcn_readlane(tabv, kb - tab_base);
        okk = phys >= 0 && phys < A.num_blocks;
        return okk ? ((size_t)phys * A.Hkv + g) * BS : 0;
    };

    typename KV::KReg kr[8];
    typename KV::template VRegs<DV> vs;
    // bias values of the lane's 8 keys, loaded one block ahead (a clamped
    // index keeps every read inside the row; out-of-range distances get 0).
    // The log-position variant has no registers to spare for that: there
    // they are loaded in the block's own step.
    constexpr bool REL_AHEAD = !LS;
    auto rel_on = [&](int jsx) { return w_lo - (jsx + 31) < A.R; };
    float rb[8];
    auto rel_fetch = [&](int jsx) {
        const int e0 = pos - (jsx + 8 * q);
#pragma unroll
        for (int i = 0; i < 8; ++i) rb[i] = relrow[min(max(e0 - i, 0), A.R - 1)];
    };
    bool ok_cur = false;
    if (ka <= kz) {
        const size_t base = block_base(ka, ok_cur);
        if (ok_cur) {
            load_k16(kr, kel + base * DQK, wid, lane);
            KV::template v_load<DV>(vs, reinterpret_cast<const char*>(vel + base * DV), wid, L - ka * BS, lane);
        }
        if (REL_AHEAD && rel_on(ka * BS + 32 * wid)) rel_fetch(ka * BS + 32 * wid);
    }
#pragma unroll 1
    for (int kb = ka; kb <= kz; ++kb) {
        const int js = kb * BS + 32 * wid;
        bool ok_next = false;
        const size_t base_next = kb < kz ? block_base(kb + 1, ok_next) : 0;
        const bool brel_next = kb < kz && rel_on(js + BS);
        if (!ok_cur) {
            bad = true;
            if (ok_next) {
                load_k16(kr, kel + base_next * DQK, wid, lane);
                KV::template v_load<DV>(vs, reinterpret_cast<const char*>(vel + base_next * DV), wid,
                                        L - (kb + 1) * BS, lane);
            }
            if (REL_AHEAD && brel_next) rel_fetch(js + BS);
            ok_cur = ok_next;
            continue;
        }
        KV::template v_store<DV>(Vw, vs, lane);
        if (ok_next)
            KV::template v_load<DV>(vs, reinterpret_cast<const char*>(vel + base_next * DV), wid, L - (kb + 1) * BS,
                                    lane);
        // S^T halves
        f32x4v S[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            S[hh] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) S[hh] = mfma16(KV::op(kr[4 * hh + st]), qreg[st], S[hh]);
        }
        if (ok_next) load_k16(kr, kel + base_next * DQK, wid, lane);
        // logits (log2 units, relative to the reference), bias, masks
        const bool brel = rel_on(js);
        const bool nmask = phantom || (js + 31 > w_lo) || (A.W > 0 && w_hi - js >= A.W);
        const int d0 = pos - (js + 8 * q);  // distance of the lane's key i is d0 - i
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = S[i >> 2][i & 3] * c1f - m_ref;
        if (brel) {
            if (!REL_AHEAD) rel_fetch(js);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int d = d0 - i;
                x[i] += (d >= 0 && d < A.R && pos >= 0) ? rb[i] * l2f : 0.f;
            }
        }
        if (REL_AHEAD && brel_next) rel_fetch(js + BS);
        if (nmask) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int d = d0 - i;
                const bool vis = d >= 0 && (A.W == 0 || d < A.W) && pos >= 0;
                x[i] = vis ? x[i] : -INFINITY;
            }
        }
        float M = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) M = fmaxf(M, x[i]);
        M = groups_max(M);
        const bool trig = (M > TAU) || (!m_set && M > -INFINITY);
        if (__any(trig)) {
            // first keys of a column set its reference; a later jump moves it
            const float delta = trig ? M : 0.f;
            const float alpha = trig ? (m_set ? __builtin_amdgcn_exp2f(-delta) : 0.f) : 1.f;
#pragma unroll
            for (int t = 0; t < DV / 16; ++t) O[t] *= alpha;
            l_sum *= alpha;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] -= delta;
            m_ref += delta;
            m_set = m_set || trig;
        }
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float pv = __builtin_amdgcn_exp2f(x[i]);
            l_sum += pv;
            pb[i] = (__bf16)pv;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < DV / 16; ++t) O[t] = mfma16(v16_operand(Vw, vrow<DV>(), t, lane), pb, O[t]);
        __builtin_amdgcn_wave_barrier();
        ok_cur = ok_next;
    }

    // Merge the four waves' partial states through LDS.
    __syncthreads();
    float* Om = reinterpret_cast<float*>(smem);   // [4][16][DV]
    float* Mm = Om + 4 * 16 * DV;                 // [4][16] reference max (or -inf)
    float* Lm = Mm + 4 * 16;                      // [4][16] row sums
    const float l_tot = groups_sum(l_sum);
    const bool any_bad = __syncthreads_or(bad);
#pragma unroll
    for (int t = 0; t < DV / 16; ++t) {
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = O[t][j];
        *reinterpret_cast<f32x4*>(Om + (wid * 16 + c) * DV + 16 * t + 4 * q) = o;
    }
    if (q == 0) {
        Mm[wid * 16 + c] = m_set ? m_ref : -INFINITY;
        Lm[wid * 16 + c] = l_tot;
    }
    __syncthreads();

    for (int e = tid; e < 16 * DV; e += 256) {
        const int col = e / DV, dv = e % DV;
        if (col >= ncols) continue;
        float mw[4], Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = Mm[w * 16 + col];
            Mx = fmaxf(Mx, mw[w]);
        }
        float den = 0.f, num = 0.f;
        if (Mx > -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = __builtin_amdgcn_exp2f(mw[w] - Mx);  // exp2(-inf) = 0
                den += f * Lm[w * 16 + col];
                num += f * Om[(w * 16 + col) * DV + dv];
            }
        }
        const int ctt = col / A.G, chl = col % A.G;
        const long long prow = ((long long)(b * A.n_q + ctt) * A.Hq + (g * A.G + chl)) * A.splits + split;
        A.part_o[prow * DV + dv] = any_bad ? NAN : (Mx > -INFINITY ? num / den * A.v_scale : 0.f);
        if (dv == 0) {
            A.part_lse[prow] = any_bad ? NAN : (Mx > -INFINITY ? (Mx + __log2f(den)) * LN2 : -INFINITY);
        }
    }
}

template <int DV, bool KV8>
__global__ void __launch_bounds__(256, 2) decode16_split_kernel(const DecodeArgs A) {
    decode16_split_body<DV, KV8, false>(A);
}

template <int DV, bool KV8>
__global__ void __launch_bounds__(256, 2) decode16_split_logpos_kernel(const DecodeArgs A) {
    decode16_split_body<DV, KV8, true>(A);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the splits: one workgroup per (row, head). Every load
// of a pair is issued before any of them is used (each thread loads up to 4
// split lse values and its first 16 partial-output values), so the merge
// costs about one memory latency rather than one per batch of splits.
// Thread (grp, d) sums dimension d over the splits grp, grp + GROUPS, ...;
// the groups are added through LDS at the end.
// ---------------------------------------------------------------------------
template <int DV>
__global__ void __launch_bounds__(256) combine_kernel(const CombineArgs A) {
    constexpr int GROUPS = 256 / DV;
    constexpr int CH = 16;  // partial outputs in flight per thread
    __shared__ float wsh[1024];
    __shared__ float red[2][4];
    __shared__ float part[GROUPS][DV];
    const int tid = threadIdx.x, wid = tid >> 6;
    const int grp = tid / DV, d = tid % DV;
    const long long pair = blockIdx.x;
    const int S = A.splits;  // <= 1024
    const float* ls = A.part_lse + pair * S;
    const float* os = A.part_o + pair * S * DV + d;

    float lv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int s = tid + 256 * k;
        lv[k] = s < S ? ls[s] : -INFINITY;
    }
    float v[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        const int s = grp + GROUPS * k;
        v[k] = s < S ? os[(long long)s * DV] : 0.f;
    }

    float M = fmaxf(fmaxf(lv[0], lv[1]), fmaxf(lv[2], lv[3]));
    const float sk = A.sink ? A.sink[pair] : -INFINITY;  // joins the normaliser with a zero value
    M = fmaxf(M, sk);
    const bool nan_here = (lv[0] != lv[0]) || (lv[1] != lv[1]) || (lv[2] != lv[2]) || (lv[3] != lv[3]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    if ((tid & 63) == 0) red[0][wid] = M;
    const bool nan_seen = __syncthreads_or(nan_here);
    M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));

    float den = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int s = tid + 256 * k;
        const float w = (s < S && M > -INFINITY) ? __builtin_amdgcn_exp2f((lv[k] - M) * LOG2E) : 0.f;
        if (s < S) wsh[s] = w;
        den += w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, 64);
    if ((tid & 63) == 0) red[1][wid] = den;
    __syncthreads();
    den = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    if (sk > -INFINITY) den += __builtin_amdgcn_exp2f((sk - M) * LOG2E);

    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        const int s = grp + GROUPS * k;
        if (s < S) acc += wsh[s] * v[k];
    }
#pragma unroll 8
    for (int s = grp + GROUPS * CH; s < S; s += GROUPS) acc += wsh[s] * os[(long long)s * DV];
    part[grp][d] = acc;
    __syncthreads();
    if (grp == 0) {
        float tot = part[0][d];
#pragma unroll
        for (int g2 = 1; g2 < GROUPS; ++g2) tot += part[g2][d];
        const float gt = A.gate ? A.gate[pair] : INFINITY;
        const float g = gt < INFINITY ? 1.f / (1.f + __builtin_amdgcn_exp2f(-gt * LOG2E)) : 1.f;
        const float inv = nan_seen ? NAN : g / den;
        A.out[pair * DV + d] = tot * inv;
        if (A.lse != nullptr && d == 0) A.lse[pair] = nan_seen ? NAN : M + logf(den);
    }
}

// ---------------------------------------------------------------------------
// Bias rows of a decode step made from the R branch ("Inkling-Small on Gaudi
// 2", "Attention with a relative bias": rel = r @ rel_logits_proj), written
// as fp32 [rows, Hq, R] for the decode kernels to read. A decode step's bias
// is rows * Hq * R floats, small next to the context it attends to, so it is
// formed by this separate small kernel rather than inside the split kernel.
// One workgroup per (256 distances, query head h, group of A.rows_per_wg
// rows; the host sizes the groups so that about one round of workgroups fills
// the GPU); lane j of wave w keeps the projection row of distance
// d0 + 64 w + j (as fp32) in registers. The group's r vectors of head h are
// staged in LDS, 64 rows at a time, and read back as broadcasts. Each bias is
// the sum over the components c, in order, of r[row, h, c] * proj[hp, d, c]:
// exact products, fp32 accumulation.
// ---------------------------------------------------------------------------
constexpr int RR_ROWS = 64;  // r rows per LDS stage

template <int DR>
__global__ void __launch_bounds__(256) rel_rows_kernel(const RelRowsArgs A) {
    __shared__ __attribute__((aligned(16))) uint16_t rs[RR_ROWS * DR];
    const int tid = threadIdx.x;
    const int h = blockIdx.y;
    const int d = blockIdx.x * 256 + tid;
    const bool live = d < A.R;
    const int hp = A.proj_heads == 1 ? 0 : h;
    // a lane past the last distance reads distance R - 1 and stores nothing
    const uint16_t* prow = A.proj + ((size_t)hp * A.R + (live ? d : A.R - 1)) * DR;
    float pf[DR];
#pragma unroll
    for (int c8 = 0; c8 < DR / 8; ++c8) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(prow + 8 * c8);
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[8 * c8 + i] = (float)v[i];
    }
    const int g0 = blockIdx.z * A.rows_per_wg, g1 = min(A.rows, g0 + A.rows_per_wg);
#pragma unroll 1
    for (int r0 = g0; r0 < g1; r0 += RR_ROWS) {
        const int nr = min(RR_ROWS, g1 - r0);
        __syncthreads();  // the previous stage's readers are done
        for (int p = tid; p < nr * (DR / 8); p += 256) {
            const int row = r0 + p / (DR / 8), c8 = p % (DR / 8);
            *reinterpret_cast<bf16x8*>(rs + (p / (DR / 8)) * DR + 8 * c8) =
                *reinterpret_cast<const bf16x8*>(A.r + ((size_t)row * A.Hq + h) * DR + 8 * c8);
        }
        __syncthreads();
#pragma unroll 2
        for (int k = 0; k < nr; ++k) {
            float acc = 0.f;
#pragma unroll
            for (int c8 = 0; c8 < DR / 8; ++c8) {
                const bf16x8 v = *reinterpret_cast<const bf16x8*>(rs + k * DR + 8 * c8);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc = fmaf((float)v[i], pf[8 * c8 + i], acc);
            }
            if (live) A.rel[((size_t)(r0 + k) * A.Hq + h) * A.R + d] = acc;
        }
    }
}

}  // namespace

namespace {

template <int DV>
void launch_tail_t(const PrefillArgs& a, dim3 g, dim3 blk, hipStream_t s) {
    if (a.kv8) {
        if (a.lscale != nullptr) hipLaunchKernelGGL((prefill_tail_fp8_logpos_kernel<DV>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((prefill_tail_fp8_kernel<DV>), g, blk, 0, s, a);
    } else {
        if (a.lscale != nullptr) hipLaunchKernelGGL((prefill_tail_logpos_kernel<DV>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((prefill_tail_kernel<DV>), g, blk, 0, s, a);
    }
}

template <int DV>
void launch_ring_t(const PrefillArgs& a, dim3 g, dim3 blk, hipStream_t s) {
    if (a.kv8) {
        if (a.lscale != nullptr) hipLaunchKernelGGL((prefill_ring_fp8_logpos_kernel<DV>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((prefill_ring_fp8_kernel<DV>), g, blk, 0, s, a);
    } else {
        if (a.lscale != nullptr) hipLaunchKernelGGL((prefill_ring_logpos_kernel<DV>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((prefill_ring_kernel<DV>), g, blk, 0, s, a);
    }
}

}  // namespace

// Kernel choice: windowed (every subtile streams bias: the ring kernel) or
// not (whole blocks, then the ring); per-row logit scale or not; bf16 or
// e4m3 K/V.
hipError_t launch_prefill(const PrefillArgs& a, int dv, hipStream_t s) {
    const long long grid = (long long)a.batch * a.n_qt * a.Hkv * a.n_hc;
    if (grid <= 0) return hipSuccess;
    const dim3 g((unsigned)grid), blk(512);
    if (a.W > 0) {
        if (dv == 128) launch_ring_t<128>(a, g, blk, s);
        else launch_ring_t<64>(a, g, blk, s);
    } else {
        if (dv == 128) launch_tail_t<128>(a, g, blk, s);
        else launch_tail_t<64>(a, g, blk, s);
    }
    return hipGetLastError();
}

namespace {

template <int DV, int DR>
void launch_relproj_t(const PrefillArgs& a, dim3 g, dim3 blk, hipStream_t s) {
    if (a.W == 0) {  // whole blocks until the first block with bias
        if (a.kv8) {
            if (a.lscale != nullptr)
                hipLaunchKernelGGL((prefill_relproj_tail_fp8_logpos_kernel<DV, DR>), g, blk, 0, s, a);
            else hipLaunchKernelGGL((prefill_relproj_tail_fp8_kernel<DV, DR>), g, blk, 0, s, a);
        } else {
            if (a.lscale != nullptr) hipLaunchKernelGGL((prefill_relproj_tail_logpos_kernel<DV, DR>), g, blk, 0, s, a);
            else hipLaunchKernelGGL((prefill_relproj_tail_kernel<DV, DR>), g, blk, 0, s, a);
        }
    } else if (a.kv8) {
        if (a.lscale != nullptr) hipLaunchKernelGGL((prefill_relproj_fp8_logpos_kernel<DV, DR>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((prefill_relproj_fp8_kernel<DV, DR>), g, blk, 0, s, a);
    } else {
        if (a.lscale != nullptr) hipLaunchKernelGGL((prefill_relproj_logpos_kernel<DV, DR>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((prefill_relproj_kernel<DV, DR>), g, blk, 0, s, a);
    }
}

template <int DV>
void launch_relproj_dv(const PrefillArgs& a, dim3 g, dim3 blk, hipStream_t s) {
    if (a.d_r == 32) launch_relproj_t<DV, 32>(a, g, blk, s);
    else if (a.d_r == 128) launch_relproj_t<DV, 128>(a, g, blk, s);
    else launch_relproj_t<DV, 64>(a, g, blk, s);
}

}  // namespace

hipError_t launch_prefill_relproj(const PrefillArgs& a, int dv, hipStream_t s) {
    const long long grid = (long long)a.batch * a.n_qt * a.Hkv * a.n_hc;
    if (grid <= 0) return hipSuccess;
    const dim3 g((unsigned)grid), blk(512);
    if (dv == 128) launch_relproj_dv<128>(a, g, blk, s);
    else launch_relproj_dv<64>(a, g, blk, s);
    return hipGetLastError();
}

namespace {

// Kernel choice for one (dv, K/V type, scale flag). G * n_q <= 16: the
// 16-column kernel (one group, n_cg == 1). dv 64 over e4m3 K/V when the grid
// fits one workgroup per CU: 8-wave workgroups (for bf16 K/V a second block
// in flight measured no faster, so the 4-wave kernel runs there). Otherwise
// the 32-column kernel.
template <int DV, bool KV8, bool LS>
void launch_split_t(const DecodeArgs& a, dim3 g, hipStream_t s) {
    const dim3 blk(256);
    if (a.G * a.n_q <= 16) {
        if (LS) hipLaunchKernelGGL((decode16_split_logpos_kernel<DV, KV8>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((decode16_split_kernel<DV, KV8>), g, blk, 0, s, a);
        return;
    }
    if constexpr (!KV8) {
        if (a.n_cg == 1 && a.G * a.n_q > 32) {  // both column groups in one workgroup
            if (LS) hipLaunchKernelGGL((decode_pair_logpos_kernel<DV>), g, dim3(512), 0, s, a);
            else hipLaunchKernelGGL((decode_pair_kernel<DV>), g, dim3(512), 0, s, a);
            return;
        }
    }
    if constexpr (DV == 64 && KV8) {
        if (a.wide) {
            if (LS) hipLaunchKernelGGL((decode_split8_logpos_kernel<DV, KV8>), g, dim3(512), 0, s, a);
            else hipLaunchKernelGGL((decode_split8_kernel<DV, KV8>), g, dim3(512), 0, s, a);
            return;
        }
    }
    if (LS) hipLaunchKernelGGL((decode_split_logpos_kernel<DV, KV8>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((decode_split_kernel<DV, KV8>), g, blk, 0, s, a);
}

template <bool LS>
void launch_split_ls(const DecodeArgs& a, int dv, dim3 g, hipStream_t s) {
    const bool kv8 = a.kv8 != 0;
    if (dv == 128) {
        if (kv8) launch_split_t<128, true, LS>(a, g, s);
        else launch_split_t<128, false, LS>(a, g, s);
    } else {
        if (kv8) launch_split_t<64, true, LS>(a, g, s);
        else launch_split_t<64, false, LS>(a, g, s);
    }
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs& a, int dv, hipStream_t s) {
    const long long grid = (long long)a.batch * a.Hkv * a.n_cg * a.splits;
    if (grid <= 0) return hipSuccess;
    const dim3 g((unsigned)grid);
    if (a.lscale != nullptr) launch_split_ls<true>(a, dv, g, s);  // per-row logit scale
    else launch_split_ls<false>(a, dv, g, s);
    return hipGetLastError();
}

// Scratch of rba_decode_noalloc (for callers that cannot allocate): the
// split partials live here instead of in a caller's workspace. Each GPU holds
// its own copy from the first launch until the process ends. In host code the
// name is only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __attribute__((aligned(256))) char scratch[RBA_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
    static std::atomic<void*> addr[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_rel_rows(const RelRowsArgs& a, hipStream_t s) {
    if (a.rows <= 0 || a.Hq <= 0 || a.R <= 0) return hipSuccess;
    if (a.rows_per_wg < 1) return hipErrorInvalidValue;
    const dim3 g((unsigned)((a.R + 255) / 256), (unsigned)a.Hq, (unsigned)((a.rows + a.rows_per_wg - 1) / a.rows_per_wg));
    const dim3 blk(256);
    if (a.d_r == 32) hipLaunchKernelGGL(rel_rows_kernel<32>, g, blk, 0, s, a);
    else if (a.d_r == 64) hipLaunchKernelGGL(rel_rows_kernel<64>, g, blk, 0, s, a);
    else if (a.d_r == 128) hipLaunchKernelGGL(rel_rows_kernel<128>, g, blk, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int dv, hipStream_t s) {
    const long long grid = a.pairs;
    if (grid <= 0) return hipSuccess;
    if (dv == 128) {
        hipLaunchKernelGGL(combine_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL(combine_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace rba
