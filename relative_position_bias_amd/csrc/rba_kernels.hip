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
//     16-key chunk: the P.V A operand (V transposed in LDS) is then one 16-byte
//     LDS read, and the lane's bias values are contiguous in the rel row.
//   * The bias is "sheared": element (column n, key j) needs rel[t_n, h_n,
//     i_n - j]. Each wave stages, per subtile, the aligned superset of its 32
//     rel row segments (32 rows x 36 floats) into LDS with 16-byte loads, then
//     every lane reads its own 16 values along the shear from LDS. Subtiles
//     whose distances are all >= R skip the rel traffic entirely; subtiles
//     that are entirely masked (causal / window) are skipped.
//   * K and V blocks (128 keys) are staged once per workgroup in LDS; V is
//     transposed on the way in (v_perm) so keys are contiguous per value dim.
//   * Online softmax in fp32 in the log2 domain with a lazy reference: the
//     reference max moves only when a block's max exceeds it by > 8 (exact
//     rearrangement; p <= 2^8), so the rescale of the accumulator is rare.
//   * Prefill: a workgroup of 8 waves shares one K/V block for up to 8 query
//     heads of one KV head (GQA packing) and 32..256 query rows.
//   * Decode: a workgroup of 4 waves shares each K/V block; wave w takes
//     subtile w, so each block is read from HBM once for all G * n_q columns;
//     splits of the block range go to different workgroups and a small
//     kernel merges them by log-sum-exp.
//   * Work-unit order puts the KV head in the fastest position of blockIdx so
//     that, with workgroups dealt round-robin to the 8 XCDs, all workgroups of
//     one KV head (which share its K/V) land on the same XCD and its L2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rba_internal.h"

namespace rba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BS = 128;        // keys per cache block
constexpr int DQK = 128;       // query/key head size
constexpr int KROW = DQK + 8;  // bf16 per LDS row of K (16-byte pad)
constexpr int VROW = BS + 8;   // bf16 per LDS row of transposed V
constexpr int RROW = 40;       // floats per LDS row of a staged rel band (36 used)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr float TAU = 8.0f;    // lazy-rescale threshold, log2 units

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

// Stage one K block (128 keys x 128 dims, bf16) into LDS with the row
// permutation the transposed-score MFMA expects: key r goes to LDS row
// (r & ~31) | perm32(r & 31).
template <int NT>
__device__ __forceinline__ void stage_k(__bf16* Ks, const uint16_t* kblk, int tid) {
#pragma unroll
    for (int it = 0; it < (BS * DQK / 8) / NT; ++it) {
        const int p = tid + NT * it;
        const int row = p >> 4, c16 = p & 15;
        const u32x4 val = *reinterpret_cast<const u32x4*>(kblk + row * DQK + c16 * 8);
        const int lrow = (row & ~31) | perm32(row & 31);
        *reinterpret_cast<u32x4*>(Ks + lrow * KROW + c16 * 8) = val;
    }
}

// Stage one V block (128 keys x DV, bf16) into LDS transposed: Vt[dv][key].
// Keys at or past `nvalid` (beyond the sequence) are written as zeros so that
// whatever the cache holds there contributes exactly 0.
template <int DV, int NT>
__device__ __forceinline__ void stage_v(__bf16* Vt, const uint16_t* vblk, int nvalid, int tid) {
    constexpr int UNITS = 32 * (DV / 8);  // units of 4 keys x 8 value dims
#pragma unroll
    for (int u0 = 0; u0 < UNITS; u0 += NT) {
        const int u = u0 + tid;
        if (UNITS % NT != 0 && u >= UNITS) break;
        const int c = u % (DV / 8), kg = u / (DV / 8);
        u32x4 in[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = 4 * kg + r;
            if (key < nvalid) {
                in[r] = *reinterpret_cast<const u32x4*>(vblk + key * DV + 8 * c);
            } else {
                in[r] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            const int qd = j >> 1;
            u32x2 o;
            o[0] = __builtin_amdgcn_perm(in[1][qd], in[0][qd], sel);
            o[1] = __builtin_amdgcn_perm(in[3][qd], in[2][qd], sel);
            *reinterpret_cast<u32x2*>(Vt + (8 * c + j) * VROW + 4 * kg) = o;
        }
    }
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

// Stage the rel values one 32-key subtile needs (rows = the wave's columns)
// into this wave's LDS band: row n holds rel[t_n, h_n, a_n .. a_n + 36) with
// a_n = floor4(pos_n - js - 31). Each lane loads float4 pieces of its own row;
// pieces outside [0, R) are zeros (distance >= R has bias 0, distance < 0 is
// masked anyway).
__device__ __forceinline__ void stage_rel(float* Rw, const float* relrow, int pos, int js, int R,
                                          int lane) {
    const int n = lane & 31, hh = lane >> 5;
    const int a_n = (pos - js - 31) & ~3;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const int c4 = hh + 2 * k;
        if (c4 < 9) {
            const int a = a_n + 4 * c4;
            f32x4 val = f32x4{0.f, 0.f, 0.f, 0.f};
            if (pos >= 0 && a >= 0 && a + 4 <= R) val = *reinterpret_cast<const f32x4*>(relrow + a);
            *reinterpret_cast<f32x4*>(Rw + n * RROW + 4 * c4) = val;
        }
    }
}

// One 32-key subtile starting at key js against the wave's 32 columns:
// QK^T on MFMA, bias along the shear, masks, online softmax, P.V on MFMA.
// `Ksub` points at the subtile's first LDS row of K, `Vsub` at its first key
// column of the transposed V.
template <int DV>
__device__ __forceinline__ void subtile(Cols<DV>& C, const __bf16* Ksub, const __bf16* Vsub,
                                        float* Rw, int js, int R, int W, float c1, int lane) {
    const int n = lane & 31, hh = lane >> 5;

    // S^T = K_sub . Q^T
    f32x16 s = zero16();
    {
        const __bf16* krow = Ksub + n * KROW + 8 * hh;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * st);
            s = mfma32(a, C.qreg[st], s);
        }
    }

    // lane holds keys js + 16 (r/8) + 8 hh + r%8 of column n
    const bool bias_on = (C.w_lo - (js + 31)) < R;
    const bool need_mask = C.phantom || (js + 31 > C.w_lo) || (W > 0 && C.w_hi - js >= W);

    float bias[16];
    if (bias_on) {
        stage_rel(Rw, C.relrow, C.pos, js, R, lane);
        __builtin_amdgcn_wave_barrier();
        const int delta = (C.pos + 1) & 3;
        const float* rb = Rw + n * RROW + (8 + delta - 8 * hh);
#pragma unroll
        for (int r = 0; r < 16; ++r) bias[r] = rb[16 * (1 - (r >> 3)) + 7 - (r & 7)];
        __builtin_amdgcn_wave_barrier();
    }

    float x[16];
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float bterm = bias_on ? fmaf(bias[r], LOG2E, -C.m_ref) : -C.m_ref;
        float t = fmaf(s[r], c1, bterm);
        if (need_mask) {
            const int key = js + 16 * (r >> 3) + 8 * hh + (r & 7);
            const bool vis = key <= C.pos && (W == 0 || C.pos - key < W);
            t = vis ? t : -INFINITY;
        }
        x[r] = t;
        M = fmaxf(M, t);
    }
    M = fmaxf(M, xor32(M));

    const bool trig = (M > TAU) || (!C.m_set && M > -INFINITY);
    if (__any(trig)) {
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

#pragma unroll
    for (int c = 0; c < 2; ++c) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(x[8 * c + i]);
            C.l_sum += p;
            pb[i] = (__bf16)p;
        }
#pragma unroll
        for (int dt = 0; dt < DV / 32; ++dt) {
            const bf16x8 va =
                *reinterpret_cast<const bf16x8*>(Vsub + (32 * dt + n) * VROW + 16 * c + 8 * hh);
            C.O[dt] = mfma32(va, pb, C.O[dt]);
        }
    }
}

template <int DV>
__device__ __forceinline__ void load_q(Cols<DV>& C, const uint16_t* qrow, bool real, int lane) {
    const int hh = lane >> 5;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        if (real) {
            C.qreg[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st + 8 * hh);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) C.qreg[st][i] = (__bf16)0.f;
        }
    }
}

template <int DV>
__device__ __forceinline__ void init_acc(Cols<DV>& C) {
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt) C.O[dt] = zero16();
    C.m_ref = 0.f;
    C.l_sum = 0.f;
    C.m_set = false;
}

// ---------------------------------------------------------------------------
// Prefill
// ---------------------------------------------------------------------------
template <int DV>
__global__ void __launch_bounds__(512) prefill_kernel(const PrefillArgs A) {
    __shared__ __attribute__((aligned(16))) __bf16 Ks[BS * KROW];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[DV * VROW];
    __shared__ __attribute__((aligned(16))) float Rs[8 * 32 * RROW];

    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, n = lane & 31;
    int id = blockIdx.x;
    const int g = id % A.Hkv;
    id /= A.Hkv;
    const int b = id % A.batch;
    id /= A.batch;
    const int hc = id % A.n_hc;
    id /= A.n_hc;
    const int qt = A.n_qt - 1 - id;  // heavy (late) tiles first

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

    Cols<DV> C;
    C.pos = real ? ctx + r : -1;
    C.relrow = A.rel + trow * A.R;
    C.w_lo = ctx + qa;
    C.w_hi = ctx + qb;
    C.phantom = qb < qa + 31;
    load_q(C, A.q + trow * DQK, real, lane);
    init_acc(C);

    const int i_lo = ctx + q0, i_hi = ctx + min(q0 + A.QT, q_len) - 1;
    const int kb_lo = A.W > 0 ? max(0, i_lo - A.W + 1) / BS : 0;
    const int kb_hi = i_hi / BS;
    float* Rw = Rs + wid * 32 * RROW;
    bool bad = false;

    for (int kb = kb_lo; kb <= kb_hi; ++kb) {
        const int phys = A.tables[(long long)b * A.max_blocks + kb];
        const bool ok = phys >= 0 && phys < A.num_blocks;
        bad = bad || !ok;
        __syncthreads();
        if (ok) {
            const size_t base = ((size_t)phys * A.Hkv + g) * BS;
            stage_k<512>(Ks, A.k + base * DQK, tid);
            stage_v<DV, 512>(Vt, A.v + base * DV, L - kb * BS, tid);
        }
        __syncthreads();
        if (!ok || !wave_active) continue;
#pragma unroll 1
        for (int sub = 0; sub < 4; ++sub) {
            const int js = kb * BS + 32 * sub;
            const bool masked_all = js > C.w_hi || (A.W > 0 && C.w_lo - (js + 31) >= A.W);
            if (masked_all) continue;
            subtile<DV>(C, Ks + 32 * sub * KROW, Vt + 32 * sub, Rw, js, A.R, A.W, A.c1, lane);
        }
    }

    if (!wave_active || !real) return;
    const float l_tot = C.l_sum + xor32(C.l_sum);
    const float inv = bad ? NAN : 1.f / l_tot;
    const int hh = lane >> 5;
    float* orow = A.out + trow * DV;
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
    if (A.lse != nullptr && hh == 0) A.lse[trow] = bad ? NAN : (C.m_ref + __log2f(l_tot)) * LN2;
}

// ---------------------------------------------------------------------------
// Split-KV decode
// ---------------------------------------------------------------------------
template <int DV>
__global__ void __launch_bounds__(256) decode_split_kernel(const DecodeArgs A) {
    // K and V staging; reused at the end for the cross-wave merge.
    __shared__ __attribute__((aligned(16))) __bf16 KV[BS * KROW + DV * VROW];
    __shared__ __attribute__((aligned(16))) float Rs[4 * 32 * RROW];
    __bf16* Ks = KV;
    __bf16* Vt = KV + BS * KROW;

    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, n = lane & 31, hh = lane >> 5;
    int id = blockIdx.x;
    const int g = id % A.Hkv;
    id /= A.Hkv;
    const int b = id % A.batch;
    id /= A.batch;
    const int cg = id % A.n_cg;
    const int split = id / A.n_cg;

    const int L = A.seq_lens[b];
    const int ncols = A.G * A.n_q;
    const int c = cg * 32 + n;
    const bool real = c < ncols;
    const int tt = real ? c / A.G : 0;
    const int hl = real ? c % A.G : 0;
    const int h = g * A.G + hl;
    const long long trow = (long long)(b * A.n_q + tt) * A.Hq + h;

    Cols<DV> C;
    C.pos = real ? L - A.n_q + tt : -1;
    C.relrow = A.rel + trow * A.R;
    const int c_hi = min(cg * 32 + 31, ncols - 1);
    C.w_lo = L - A.n_q + (cg * 32) / A.G;
    C.w_hi = L - A.n_q + c_hi / A.G;
    C.phantom = c_hi < cg * 32 + 31;
    load_q(C, A.q + trow * DQK, real, lane);
    init_acc(C);

    const int nb = (L + BS - 1) / BS;
    const int kb_first = A.W > 0 ? max(0, (L - A.n_q) - A.W + 1) / BS : 0;
    const int s_lo = kb_first + split * A.bps;
    const int s_hi = min(s_lo + A.bps, nb);
    float* Rw = Rs + wid * 32 * RROW;
    bool bad = false;

    for (int kb = s_lo; kb < s_hi; ++kb) {
        const int phys = A.tables[(long long)b * A.max_blocks + kb];
        const bool ok = phys >= 0 && phys < A.num_blocks;
        bad = bad || !ok;
        __syncthreads();
        if (ok) {
            const size_t base = ((size_t)phys * A.Hkv + g) * BS;
            stage_k<256>(Ks, A.k + base * DQK, tid);
            stage_v<DV, 256>(Vt, A.v + base * DV, L - kb * BS, tid);
        }
        __syncthreads();
        if (!ok) continue;
        const int js = kb * BS + 32 * wid;
        const bool masked_all = js > C.w_hi || (A.W > 0 && C.w_lo - (js + 31) >= A.W);
        if (masked_all) continue;
        subtile<DV>(C, Ks + 32 * wid * KROW, Vt + 32 * wid, Rw, js, A.R, A.W, A.c1, lane);
    }

    // Merge the four waves' partial states through LDS.
    __syncthreads();
    float* Om = reinterpret_cast<float*>(KV);   // [4][32][DV]
    float* Mm = Rs;                             // [4][32] reference max (or -inf)
    float* Lm = Rs + 4 * 32;                    // [4][32] row sums
    const float l_tot = C.l_sum + xor32(C.l_sum);
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

    // 32 columns x DV values over 256 threads
    for (int e = tid; e < 32 * DV; e += 256) {
        const int col = e / DV, dv = e % DV;
        const int cc = cg * 32 + col;
        if (cc >= ncols) continue;
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = Mm[w * 32 + col];
            M = fmaxf(M, mw[w]);
        }
        float den = 0.f, num = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = __builtin_amdgcn_exp2f(mw[w] - M);  // exp2(-inf) = 0
                den += f * Lm[w * 32 + col];
                num += f * Om[(w * 32 + col) * DV + dv];
            }
        }
        const int ctt = cc / A.G, chl = cc % A.G;
        const long long prow = ((long long)(b * A.n_q + ctt) * A.Hq + (g * A.G + chl)) * A.splits + split;
        const float o = bad ? NAN : (M > -INFINITY ? num / den : 0.f);
        A.part_o[prow * DV + dv] = o;
        if (dv == 0) {
            A.part_lse[prow] = bad ? NAN : (M > -INFINITY ? (M + __log2f(den)) * LN2 : -INFINITY);
        }
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the splits: one wave per (row, head).
// ---------------------------------------------------------------------------
template <int DV>
__global__ void __launch_bounds__(256) combine_kernel(const CombineArgs A) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long pair = (long long)blockIdx.x * 4 + wid;
    if (pair >= A.pairs) return;
    const float* ls = A.part_lse + pair * A.splits;
    const float* os = A.part_o + pair * A.splits * DV;

    float M = -INFINITY;
    for (int s = lane; s < A.splits; s += 64) M = fmaxf(M, ls[s]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    bool nan_seen = false;
    for (int s = lane; s < A.splits; s += 64) nan_seen = nan_seen || (ls[s] != ls[s]);
    nan_seen = __any(nan_seen);

    constexpr int PER = DV / 64;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
    float den = 0.f;
    if (M > -INFINITY) {
        for (int s = 0; s < A.splits; ++s) {
            const float w = __builtin_amdgcn_exp2f((ls[s] - M) * LOG2E);
            den += w;
#pragma unroll
            for (int k = 0; k < PER; ++k) acc[k] += w * os[s * DV + lane + 64 * k];
        }
    }
    const float inv = nan_seen ? NAN : 1.f / den;
#pragma unroll
    for (int k = 0; k < PER; ++k) A.out[pair * DV + lane + 64 * k] = acc[k] * inv;
    if (A.lse != nullptr && lane == 0) A.lse[pair] = nan_seen ? NAN : M + logf(den);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int dv, hipStream_t s) {
    const long long grid = (long long)a.batch * a.n_qt * a.Hkv * a.n_hc;
    if (grid <= 0) return hipSuccess;
    if (dv == 128) {
        hipLaunchKernelGGL(prefill_kernel<128>, dim3((unsigned)grid), dim3(512), 0, s, a);
    } else {
        hipLaunchKernelGGL(prefill_kernel<64>, dim3((unsigned)grid), dim3(512), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs& a, int dv, hipStream_t s) {
    const long long grid = (long long)a.batch * a.Hkv * a.n_cg * a.splits;
    if (grid <= 0) return hipSuccess;
    if (dv == 128) {
        hipLaunchKernelGGL(decode_split_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL(decode_split_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int dv, hipStream_t s) {
    const long long grid = ((long long)a.pairs + 3) / 4;
    if (grid <= 0) return hipSuccess;
    if (dv == 128) {
        hipLaunchKernelGGL(combine_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL(combine_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace rba
