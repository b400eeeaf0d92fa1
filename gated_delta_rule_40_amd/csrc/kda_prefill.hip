// kda_prefill.hip -- chunked KDA prefill for gfx950.
//
// The recurrence (page "Kimi K3 把 3T 级模型、百万上下文和 Agent 训练接成一套系统",
// ailearn.mscapital.top/kimi-k3.html, card "KDA 单头递归"), per (sequence, head):
//     S_t = (I - b_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t.
//
// Chunked form evaluated here (derived from that recurrence; C tokens per
// chunk, entering state S0, Gamma_r = sum_{i<=r} g_i, all per key channel):
//     X   = Diag(b) (V - K+ S0)                           K+ = K (.) e^Gamma
//     W   = (I + N)^-1 X,     N = Diag(b) A,  A_ri = sum_c k_rc k_ic e^(Gamma_rc - Gamma_ic), i < r
//     O   = Q+ S0 + P W,      P_ri = sum_c q_rc k_ic e^(Gamma_rc - Gamma_ic), i <= r
//     S_C = Diag(e^Gamma_C) S0 + K^T W                    K^ = K (.) e^(Gamma_C - Gamma)
// A and P ("Gram" tiles) factor each decay e^(Gamma_r - Gamma_i) into a row and
// a column factor.  When every channel decays by at most e^-11 over the chunk
// (always true for gates of a few tenths), the chunk start is the reference:
// rows use K+ / Q+ and columns K (.) e^-Gamma <= e^11, so A and P are plain
// dense products of the operands the chain uses anyway.  Otherwise the factors
// are referenced to 16-token sub-tile boundaries (card "g ∈ (-5, 0)": inside a
// 16-token tile the cumulative scaling stays within bf16 range) and the Gram
// runs on fp32 MFMA, so g anywhere in [-5, 0] stays exact.
//
// Precision (bf16 q/k/v): every MFMA operand is fp16 with fp32 accumulation;
// the fp32 state, X and W are converted with exact per-column power-of-two
// scales, so their range is unrestricted; (I + N)^-1 is kept per 16x16 block
// with a power-of-two scale.  fp32 q/k/v use fp32 MFMA throughout.
//
// Work decomposition: one workgroup per (sequence, head, block of BV value
// columns), NW = BV/16 waves.  Each wave owns 16 columns of the fp32 state,
// kept in MFMA accumulator registers for the whole sequence.  Per chunk:
//   1. decay prep from registers loaded one chunk ahead: sub-tile gate sums,
//      per-token decay products, decayed operands to LDS;
//   2. Gram tiles A, P on MFMA (jobs spread over the waves);
//   3. (I + N)^-1: 16x16 diagonal blocks by VALU forward substitution, then
//      off-diagonal blocks by block recursion on MFMA;
//   4. state-dependent chain per wave: X, W, O and the state update on MFMA;
//   5. coalesced store of the output tile.
// Ragged chunks are zero-padded (k = q = v = 0, g = 0, b = 0), which leaves
// the result exact.
//
// Two-stage form (context-parallel entry): phases 1-3 do not depend on the
// state, so a chunk-parallel pass (MODE_PREP) runs them once per (chunk,
// head) and stores the chain operands as a chunk image; kda_chain_kernel then
// runs phase 4 alone per (segment, head, value block), reading the images.
// Segments are combined through their end state from zero and transition
// (page card "传固定状态片段": local cumulative transform plus zero-state
// fragment, then a prefix combination).
#include <type_traits>

#include "kda_device.hpp"

namespace kda {

constexpr int DK = 128;
constexpr int SUB = 16;

template <typename TIn, int C, int NW>
struct PrefillCfg {
    static constexpr bool kIn16 = !std::is_same<TIn, float>::value;
    typedef typename std::conditional<kIn16, f16_t, float>::type OpT;   // MFMA operands
    static constexpr int BV = 16 * NW;
    static constexpr int NT = 64 * NW;
    static constexpr int NSUB = C / SUB;
    static constexpr int NPAIR = NSUB * (NSUB + 1) / 2;
    static constexpr int KB = Mma<OpT>::KB;
    static_assert(C % KB == 0, "chunk must be a multiple of the MFMA K-block");
    static_assert(NSUB >= 1 && NSUB <= 4, "chunk of 16..64 tokens");
    // Decay products are built from fixed 4-token groups, always combined in
    // the same order, so every tiling computes bit-identical decay factors.
    static constexpr int GRP = 4;
    static constexpr int NGRP = C / GRP;
    // fast decay prep: thread -> (segment of SEG tokens, CPI consecutive
    // channels), from registers loaded one chunk ahead (ITEMS items per thread)
    static constexpr int CPI = 4;
    static constexpr int IPR = DK / CPI;                               // items per token row
    static constexpr int SEG0 = C * IPR / NT;
    static constexpr int SEG = SEG0 < GRP ? GRP : (SEG0 > 16 ? 16 : SEG0);
    static constexpr int NSEG = C / SEG;
    static constexpr int ITEMS = (NSEG * IPR + NT - 1) / NT;
    static_assert(SEG % GRP == 0 && SUB % SEG == 0, "prep mapping");
    // slow decay prep: thread -> (sub-tile, CPT consecutive channels)
    static constexpr int CPT = (DK * NSUB >= NT) ? DK * NSUB / NT : 1;
    static constexpr int NPREP = DK * NSUB / CPT;                      // slow prep threads
    static_assert(CPT == 1 || CPT == 2 || CPT == 4, "channels per prep thread");
    // chunk-start reference allowed when no channel decays by more than this
    // over the chunk (11 for fp16 operands, 60 for fp32)
    static constexpr float SPAN_CHUNK = kIn16 ? 11.f : 60.f;
    // exact power-of-two rebalance of fp16 operands: row operands x GS, column /GS
    static constexpr float GS = kIn16 ? 32.f : 1.f;

    // row strides (elements), rows padded by 16 bytes against bank conflicts
    static constexpr int LDK = DK + 16 / (int)sizeof(OpT);     // [C][DK] operand tiles
    static constexpr int LDC = C + 16 / (int)sizeof(OpT);      // [*][C] operand tiles
    static constexpr int LDK32 = DK + 4;                       // [C][DK] fp32 Gram inputs
    static constexpr int LDV = BV + 16 / (int)sizeof(TIn);     // value / output tiles

    // Rows of the 2-byte MFMA row operands (NKp, Qp, Kc along channels; KhT, P
    // along tokens) hold their contraction index in kperm order, so each lane
    // reads a K-block fragment with one 16-byte load.
    static constexpr size_t tileK = sizeof(OpT) * C * LDK;
    // region 0: chain operands and staging; the fp32 sub-tile Gram inputs of a
    // strong-decay chunk overlay it (everything but Kc is rewritten afterwards)
    static constexpr size_t offNKp = 0;                                    // -GS K+   [C][LDK]
    static constexpr size_t offQp = offNKp + tileK;                        //  GS Q+   [C][LDK]
    static constexpr size_t offKc = offQp + tileK;                         //  K e^-G / GS [C][LDK]
    static constexpr size_t offKhT = offKc + tileK;                        //  GS K^T  [DK][LDC]
    static constexpr size_t offV = offKhT + sizeof(OpT) * DK * LDC;        //  V       [C][LDV]
    static constexpr size_t offO = offV + sizeof(TIn) * C * LDV;           //  O       [C][LDV]
    static constexpr size_t endFast = offO + sizeof(TIn) * C * LDV;
    static constexpr size_t offKr32 = 0;
    static constexpr size_t offQr32 = offKr32 + sizeof(float) * C * LDK32;
    static constexpr size_t offKD32 = offQr32 + sizeof(float) * C * LDK32;
    static constexpr size_t endSlow = offKD32 + sizeof(float) * C * LDK32;
    static constexpr size_t end0 = ((endFast > endSlow ? endFast : endSlow) + 15) / 16 * 16;
    // region 1: Gram outputs and (I + N)^-1
    static constexpr int LDAD = 20;                                          // 80-byte rows
    static constexpr size_t offAd = end0;                                   // fp32 [NSUB][16][LDAD], N^T
    static constexpr size_t offN = offAd + sizeof(float) * NSUB * SUB * LDAD; // OpT [C][LDC]
    static constexpr size_t offT = offN + sizeof(OpT) * C * LDC;            // OpT [C][LDC]
    static constexpr size_t offP = offT + sizeof(OpT) * C * LDC;            // OpT [C][LDC]
    static constexpr size_t end1 = (offP + sizeof(OpT) * C * LDC + 15) / 16 * 16;
    // small fp32 tables
    static constexpr size_t offF = end1;                                    // [NGRP][DK]
    static constexpr size_t offH = offF + sizeof(float) * NGRP * DK;        // [NPAIR][DK]
    static constexpr size_t offGam = offH + sizeof(float) * NPAIR * DK;     // [DK]
    static constexpr size_t offBeta = offGam + sizeof(float) * DK;          // [C]
    static constexpr size_t offTs = offBeta + sizeof(float) * C;            // [NSUB][NSUB]
    static constexpr size_t offPre = offTs + (sizeof(float) * NSUB * NSUB + 15) / 16 * 16;   // [NGRP + 1][DK]
    static constexpr size_t bytes = offPre + sizeof(float) * (NGRP + 1) * DK;
    static_assert(bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
    // workgroups per CU that the LDS allows (the register budget is set to match)
    static constexpr int WG_PER_CU = (2 * bytes <= 160 * 1024) ? 2 : 1;
    // waves per SIMD the register budget is sized for (at most 2: 256 registers)
    static constexpr int WAVES_PER_EU = (WG_PER_CU * NW) / 4 >= 2 ? 2 : 1;
};

// Segmented (context-parallel) execution.  A plan lists segments of the
// packed sequences as {sequence, first token, end token, flags}; entries with
// sequence < 0 are unused.  SEG_SUMMARY runs each segment from a zero state
// over dv value columns plus DK transition columns (V = 0, entering state I)
// and writes [S_end | transition]; SEG_OUTPUT runs each segment from its
// entering state (seg_init) and writes outputs and, for a last segment, the
// final state.
enum { SEG_OUTPUT = 0, SEG_SUMMARY = 1 };
struct SegArgs {
    const int32_t *plan;     // [num_segs][4] or nullptr (one unit per sequence)
    int32_t num_segs;
    int32_t mode;            // SEG_OUTPUT or SEG_SUMMARY
    const float *seg_init;   // [num_segs][H][DK][dv] entering states (SEG_OUTPUT)
    float *seg_out;          // [num_segs][H][DK][dv + DK] summaries (SEG_SUMMARY)
    const int32_t *chunk_off;   // [N + 1] first chunk of each sequence (chunk-image passes)
    f32x4 *img;                 // chunk-operand images (chunk-image passes)
    float *snap;                // [N][max_snaps][H][DK][dv] state snapshots, or nullptr (fused kernel)
    int32_t snap_every;         // tokens between snapshots, a multiple of the chunk
    int32_t max_snaps;
    const int32_t *sched;       // [num_segs] plan index of each dispatch position, or nullptr (plan order)
    // entering states indexed by summary unit instead of segment (SEG_OUTPUT):
    // a segment starting t tokens into sequence n reads seg_init entry
    // init_seq_seg[n] + t / init_unit (segments start on unit boundaries), or
    // nullptr (entry = segment index)
    const int32_t *init_seq_seg;
    int32_t init_unit, init_units;
    int32_t prep_group;         // chunk-operand pass: consecutive chunks per workgroup (1 .. PREP_GROUP)
    int32_t img_slots;          // chunk-operand pass: image slots per head (> chunks of valid input)
};

// seg_init entry of plan segment su (sequence n, first token t_start)
__device__ __forceinline__ int64_t seg_init_entry(const SegArgs &seg, int su, int n, int t_start,
                                                  const int32_t *cu_seqlens, int32_t total_tokens)
{
    if (!seg.init_seq_seg) return su;
    const int seq_start = min(max(cu_seqlens[n], 0), total_tokens);
    const int64_t e = (int64_t)seg.init_seq_seg[n] + max(t_start - seq_start, 0) / seg.init_unit;
    return min(max(e, (int64_t)0), (int64_t)seg.init_units - 1);
}

enum { MODE_FUSED = 0, MODE_PREP = 1, MODE_SNAP = 2 };   // MODE_SNAP: fused + state snapshots
constexpr int PREP_GROUP = 8;    // most consecutive chunks per workgroup of the chunk-operand pass

// Chunk-operand image: everything the state chain of one (chunk, head) reads
// besides V, as computed by the chunk-operand pass -- -GS K+, GS K^
// transposed, the (I + N)^-1 blocks, the fp32 chunk decay, beta and T-block
// scales (what a segment summary needs: the first NVEC_SUM vectors), then
// GS Q+ and P (for the outputs).  Packed row-major without padding as 16-byte
// vectors; lds_off maps vector v to its place in an LDS buffer that uses the
// padded strides of PrefillCfg.  Chunks are numbered across the
// packed sequences: sequence n owns chunks chunk_off[n] .. chunk_off[n+1]-1,
// and the image of (chunk c, head h) is vector block c * H + h.
template <typename TIn, int C>
struct ChunkImage {
    typedef PrefillCfg<TIn, C, 4> P;                   // strides (independent of NW)
    typedef typename P::OpT OpT;
    static constexpr int EPV = 16 / (int)sizeof(OpT);  // elements per vector
    static constexpr int NSUB = C / SUB;
    static constexpr int vNKp = C * DK / EPV, vQp = C * DK / EPV, vKhT = DK * C / EPV;
    static constexpr int vT = C * C / EPV, vP = C * C / EPV;
    static constexpr int vGam = DK / 4, vBeta = C / 4, vTs = (NSUB * NSUB + 3) / 4;
    static constexpr int NVEC_SUM = vNKp + vKhT + vT + vGam + vBeta + vTs;
    static constexpr int NVEC = NVEC_SUM + vQp + vP;
    static constexpr size_t BYTES = (size_t)NVEC * 16;
    struct Offs { uint32_t nkp, qp, kht, t, p, gam, beta, ts; };   // byte offsets of the regions
    __device__ static __forceinline__ uint32_t lds_off(int v, const Offs &o) {
        constexpr int RK = DK / EPV, RC = C / EPV;                  // vectors per row
        constexpr uint32_t E = sizeof(OpT);
        if (v < vNKp) return o.nkp + ((v / RK) * P::LDK + (v % RK) * EPV) * E;
        v -= vNKp;
        if (v < vKhT) return o.kht + ((v / RC) * P::LDC + (v % RC) * EPV) * E;
        v -= vKhT;
        if (v < vT) return o.t + ((v / RC) * P::LDC + (v % RC) * EPV) * E;
        v -= vT;
        if (v < vGam) return o.gam + 16 * v;
        v -= vGam;
        if (v < vBeta) return o.beta + 16 * v;
        v -= vBeta;
        if (v < vTs) return o.ts + 16 * v;
        v -= vTs;
        if (v < vQp) return o.qp + ((v / RK) * P::LDK + (v % RK) * EPV) * E;
        return o.p + (((v - vQp) / RC) * P::LDC + ((v - vQp) % RC) * EPV) * E;
    }
};

// 16-byte vectors of the 4-aligned tails below the diagonal of columns
// s0 .. s1-1 of a 16 x 16 block (rows ((s + 1) & ~3) .. 15 of column s).
constexpr int tail_vecs(int s0, int s1) {
    int n = 0;
    for (int s = s0; s < s1; ++s) n += (SUB - ((s + 1) & ~3)) / 4;
    return n;
}

// sub-tile pair p -> (a, b), b <= a
__device__ __forceinline__ void pair_of(int p, int &a, int &b) {
    a = 0;
    while ((a + 1) * (a + 2) / 2 <= p) ++a;
    b = p - a * (a + 1) / 2;
}

// Gram tiles A (strictly lower) and P (lower incl.), one job = one sub-tile
// pair and one of the two products.  Operands of type GT with row stride ld;
// if hs != nullptr the column operand of pair p is scaled per channel by
// hs[p][.].  sign: +1 if the row operand of A is +K, -1 if it holds -K.
// Output: N = Diag(beta) A (diagonal blocks fp32 to sAd, others to sN) and P.
template <typename GT, typename OpT, int C, int NW>
__device__ __forceinline__ void gram_tiles(const GT *rowA_base, const GT *rowP_base, const GT *col_base,
                                           int ld, const float *hs, float signA,
                                           const float *sBeta, float *sAd, OpT *sN, OpT *sP, int ldc,
                                           int wave, int lj, int lm)
{
    typedef Mma<GT> G;
    constexpr int NSUB = C / SUB, NPAIR = NSUB * (NSUB + 1) / 2;
    constexpr int KBc = Mma<OpT>::KB;    // K-block of the P W contraction in the chain
    for (int job = wave; job < 2 * NPAIR; job += NW) {
        const int p = job >> 1;
        const bool isP = job & 1;
        int a, b;
        pair_of(p, a, b);
        f32x4 acc = zero4();
        const GT *rowR = (isP ? rowP_base : rowA_base) + (a * SUB + lm) * ld;
        const GT *rowC = col_base + (b * SUB + lm) * ld;
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += G::KB) {
            const typename G::frag bf = hs ? G::load_scaled(rowC, hs + p * DK, k0, lj) : G::load_p(rowC, k0, lj);
            acc = G::mma(G::load_p(rowR, k0, lj), bf, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = 4 * lj + i;                 // row within sub-tile a
            const int r = a * SUB + rl, cc = b * SUB + lm;
            if (isP) {
                const float pv = (a == b && lm > rl) ? 0.f : acc[i];
                sP[r * ldc + kperm<OpT>(cc)] = from_f<OpT>(pv);
                if (KBc == 32 && a == b && (a & 1) == 0 && a + 1 < NSUB)
                    sP[r * ldc + kperm<OpT>(cc + SUB)] = from_f<OpT>(0.f);  // a K-block pairs sub-tiles a, a+1
            } else if (a != b) {
                sN[r * ldc + cc] = from_f<OpT>(sBeta[r] * signA * acc[i]);   // N = Diag(beta) A
            }
        }
        if (!isP && a == b) {
            // diagonal block, strictly lower, stored transposed: sAd[a][col][row]
            f32x4 nt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 4 * lj + i;
                nt[i] = (lm >= rl) ? 0.f : sBeta[a * SUB + rl] * signA * acc[i];
            }
            *reinterpret_cast<f32x4 *>(sAd + (a * SUB + lm) * 20 + 4 * lj) = nt;
        }
    }
}

// B operand of a 16-wide contraction read from a row-major OpT tile:
// B[k][n] = tile[k][n], lane (n + 16 j) takes rows 4j..4j+3 of column n.
template <typename OpT>
__device__ __forceinline__ typename Mma<OpT>::frag16 load16_col(const OpT *tile, int ld, int lj, int lm) {
    typename Mma<OpT>::frag16 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = tile[(4 * lj + e) * ld + lm];
    return r;
}

// Decayed operands of a strong-decay chunk, with 16-token sub-tile references,
// reading the chunk from global memory (it is not staged for this path).
// gram_inputs: fp32 Gram inputs K (.) R, Q (.) R, K (.) D with R, D the decay
// products inside the sub-tile up to / after each token; otherwise the chain
// operands -GS K+, GS Q+, GS K^T.  Written as plain loops that hold few values
// at a time, so that this rarely used path adds little register pressure.
template <typename TIn, int C, int NW>
__device__ __forceinline__ void prep_slow(
    bool gram_inputs, const TIn *__restrict__ q, const TIn *__restrict__ k, const float *__restrict__ g,
    int c0, int L, int64_t rowK, int64_t hK, int tid, const float *sF, float *sKr32, float *sQr32,
    float *sKD32, typename PrefillCfg<TIn, C, NW>::OpT *sNKp, typename PrefillCfg<TIn, C, NW>::OpT *sQp,
    typename PrefillCfg<TIn, C, NW>::OpT *sKhT)
{
    typedef PrefillCfg<TIn, C, NW> P;
    typedef typename P::OpT OpT;
    constexpr int CPT = P::CPT, NGRP = P::NGRP, GPS = SUB / P::GRP;
    constexpr int LDK = P::LDK, LDC = P::LDC, LDK32 = P::LDK32;
    constexpr float GS = P::GS;
    if (tid >= P::NPREP) return;
    const int pa = tid / (DK / CPT), pc = (tid % (DK / CPT)) * CPT;
#pragma unroll 1
    for (int e = 0; e < CPT; ++e) {
        const int c = pc + e;
        float erho = 1.f, suff = 1.f;
        for (int s = 0; s < pa * GPS; ++s) erho *= sF[s * DK + c];
        for (int s = (pa + 1) * GPS; s < NGRP; ++s) suff *= sF[s * DK + c];
        float D = 1.f;                      // prod of alpha after r within the sub-tile
#pragma unroll 1
        for (int rr = SUB - 1; rr >= 0; --rr) {
            const int r = pa * SUB + rr;
            const bool ok = r < L;
            const int64_t off = (int64_t)(c0 + min(r, L - 1)) * rowK + hK + c;
            const float kv = ok ? to_f(k[off]) : 0.f;
            if (gram_inputs) sKD32[r * LDK32 + c] = kv * D;
            else sKhT[c * LDC + kperm<OpT>(r)] = from_f<OpT>(GS * kv * D * suff);
            D *= ok ? __expf(g[off]) : 1.f;
        }
        float R = 1.f;                      // prod of alpha up to r within the sub-tile
#pragma unroll 1
        for (int rr = 0; rr < SUB; ++rr) {
            const int r = pa * SUB + rr;
            const bool ok = r < L;
            const int64_t off = (int64_t)(c0 + min(r, L - 1)) * rowK + hK + c;
            const float kv = ok ? to_f(k[off]) : 0.f, qv = ok ? to_f(q[off]) : 0.f;
            R *= ok ? __expf(g[off]) : 1.f;
            if (gram_inputs) {
                sKr32[r * LDK32 + c] = kv * R;
                sQr32[r * LDK32 + c] = qv * R;
            } else {
                sNKp[r * LDK + kperm<OpT>(c)] = from_f<OpT>(-GS * kv * R * erho);
                sQp[r * LDK + kperm<OpT>(c)] = from_f<OpT>(GS * qv * R * erho);
            }
        }
    }
}

// Largest per-column state scale (2^64; see chain_chunk).
constexpr float kScaleCap = 18446744073709551616.f;

// State-dependent part of one chunk for the 16 value columns of this wave:
//     X = Diag(b) (V - K+ S0),  W = (I + N)^-1 X,  O = Q+ S0 + P W,
//     S = Diag(e^Gamma_C) S0 + K^T W,
// reading the chunk operands from LDS (sNKp = -GS K+, sQp = GS Q+,
// sKhT = GS K^ transposed, sT = (I + N)^-1 blocks with scales sTs, sP, the
// chunk decay sGam and sBeta), V from sV[r * ldv + vc] and writing O to
// sO[r * ldo + oc] unless SUMMARY.
//
// S (this wave's 128 x 16 slice, MFMA accumulator layout) holds the state
// scaled per column, S~ = S * sS, with sS an exact power of two per lane's
// column (always 1 for fp32 operands).  S~ then feeds the fp16 MFMA operand
// with no per-chunk multiply, and the update runs as the MFMA accumulator:
// W is rounded as W sS / GS, so (GS K^)^T (W sS / GS) = K^T W sS lands in the
// same scaled units.  sS changes (by exact powers of two) only when a column
// leaves [2^-8, 2^15), or when W sS / GS would leave the fp16 range.
template <typename TIn, int C, int ldv, int ldo, bool SUMMARY, int NCT = 1>
__device__ __forceinline__ void chain_chunk(
    f32x4 (&S)[NCT][DK / 16], float (&sS)[NCT], const typename PrefillCfg<TIn, C, 4>::OpT *sNKp,
    const typename PrefillCfg<TIn, C, 4>::OpT *sQp, const typename PrefillCfg<TIn, C, 4>::OpT *sKhT,
    const typename PrefillCfg<TIn, C, 4>::OpT *sT, const typename PrefillCfg<TIn, C, 4>::OpT *sP,
    const float *sTs, const float *sGam, const float *sBeta, const TIn *sV, int vc, TIn *sO, int oc,
    int lj, int lm)
{
    // NCT column tiles of 16 per wave (tile ct: value column vc + 16 ct, output column oc + 16 ct):
    // every operand fragment read from LDS serves all of them
    typedef PrefillCfg<TIn, C, 4> P;
    typedef typename P::OpT OpT;
    typedef Mma<OpT> M;
    constexpr bool kIn16 = P::kIn16;
    constexpr int NSUB = P::NSUB, KB = P::KB, LDK = P::LDK, LDC = P::LDC;
    constexpr float GS = P::GS;

    float isS[NCT];
    typename M::frag Sf[NCT][DK / KB];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        isS[ct] = pow2_inv(sS[ct]) * (1.f / GS);   // undoes the state scale and the GS on K+ / Q+
#pragma unroll
        for (int kb = 0; kb < DK / KB; ++kb) Sf[ct][kb] = M::from_acc(&S[ct][kb * (KB / 16)]);
    }

    // X = Diag(beta) (V - K+ S0)       (rows of sNKp hold -GS K+)
    f32x4 X[NCT][NSUB];
    float xmax[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) xmax[ct] = 0.f;
#pragma unroll
    for (int mt = 0; mt < NSUB; ++mt) {
        f32x4 t[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) t[ct] = zero4();
        const OpT *rowA = sNKp + (mt * SUB + lm) * LDK;
#pragma unroll
        for (int kb = 0; kb < DK / KB; ++kb) {
            const typename M::frag af = M::load_p(rowA, kb * KB, lj);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) t[ct] = M::mma(af, Sf[ct][kb], t[ct]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = mt * SUB + 4 * lj + i;
            const float br = sBeta[r];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                X[ct][mt][i] = br * (to_f(sV[r * ldv + vc + 16 * ct]) + t[ct][i] * isS[ct]);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) xmax[ct] = absmax_acc(xmax[ct], X[ct][mt]);
    }
    // W = (I + N)^-1 X, block lower triangular, per-block scales
    typename M::frag16 X16[NCT][NSUB];
    float isX[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        float sX = 1.f;
        if (kIn16) sX = pow2_scale(colmax(xmax[ct]));
        isX[ct] = pow2_inv(sX);
#pragma unroll
        for (int b = 0; b < NSUB; ++b) X16[ct][b] = M::from_acc16(X[ct][b], sX);
    }
    f32x4 W[NCT][NSUB];
    float wmax[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) wmax[ct] = 0.f;
#pragma unroll
    for (int a = 0; a < NSUB; ++a) {
        f32x4 w[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) w[ct] = zero4();
        const OpT *rowT = sT + (a * SUB + lm) * LDC;
#pragma unroll
        for (int b = 0; b <= a; ++b) {
            const typename M::frag16 tf = M::load16(rowT, b * SUB, lj);
            const float ts = sTs[a * NSUB + b];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) w[ct] += M::mma16(tf, X16[ct][b], zero4()) * (ts * isX[ct]);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            W[ct][a] = w[ct];
            wmax[ct] = absmax_acc(wmax[ct], w[ct]);
        }
    }
    // W enters in the state's units; if W sS / GS would not fit fp16, the
    // state scale comes down first (wave-uniform branch, rarely taken)
    typename M::frag Wf[NCT][C / KB];
    float isWt[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        float sWt = sS[ct] * (1.f / GS);
        if (kIn16) {
            const float wm = colmax(wmax[ct]) * sWt;
            const float p = wm >= 32768.f ? pow2_scale(wm) : 1.f;
            if (__ballot(p != 1.f)) {
#pragma unroll
                for (int r = 0; r < DK / 16; ++r) S[ct][r] *= p;
                sS[ct] *= p;
                sWt *= p;
            }
        }
        isWt[ct] = pow2_inv(sWt);
#pragma unroll
        for (int kb = 0; kb < C / KB; ++kb) Wf[ct][kb] = M::from_acc(&W[ct][kb * (KB / 16)], sWt);
    }

    // O = Q+ S0 + P W       (rows of sQp hold GS Q+; Sf carries the entry scale)
#pragma unroll
    for (int mt = 0; mt < (SUMMARY ? 0 : NSUB); ++mt) {
        f32x4 o1[NCT], o2[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) o1[ct] = o2[ct] = zero4();
        const OpT *rowQ = sQp + (mt * SUB + lm) * LDK;
#pragma unroll
        for (int kb = 0; kb < DK / KB; ++kb) {
            const typename M::frag qf = M::load_p(rowQ, kb * KB, lj);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) o1[ct] = M::mma(qf, Sf[ct][kb], o1[ct]);
        }
        const OpT *rowP = sP + (mt * SUB + lm) * LDC;
#pragma unroll
        for (int kb = 0; kb < C / KB; ++kb)
            if (kb * KB <= mt * SUB + SUB - 1) {
                const typename M::frag pf = M::load_p(rowP, kb * KB, lj);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) o2[ct] = M::mma(pf, Wf[ct][kb], o2[ct]);
            }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const f32x4 o = o1[ct] * isS[ct] + o2[ct] * isWt[ct];
#pragma unroll
            for (int i = 0; i < 4; ++i) sO[(mt * SUB + 4 * lj + i) * ldo + oc + 16 * ct] = from_f<TIn>(o[i]);
        }
    }
    // S~ = Diag(gamma) S~ + (GS K^)^T Wf, the decayed state as the accumulator
    float smax[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) smax[ct] = 0.f;
#pragma unroll
    for (int r = 0; r < DK / 16; ++r) {
        const f32x4 gm = *reinterpret_cast<const f32x4 *>(sGam + 16 * r + 4 * lj);
        f32x4 t[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) t[ct] = S[ct][r] * gm;
        const OpT *rowK = sKhT + (16 * r + lm) * LDC;
#pragma unroll
        for (int kb = 0; kb < C / KB; ++kb) {
            const typename M::frag kf = M::load_p(rowK, kb * KB, lj);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) t[ct] = M::mma(kf, Wf[ct][kb], t[ct]);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            S[ct][r] = t[ct];
            if (kIn16) smax[ct] = absmax_acc(smax[ct], t[ct]);
        }
    }
    // keep every column inside [2^-8, 2^15) (fp16 normal range with margin);
    // the scale never grows past 2^64: a column decaying towards zero (the
    // transition columns of a strongly decaying segment) is then left to
    // shrink, its values being negligible at that point
    if (kIn16) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const float m = colmax(smax[ct]);
            float q = 1.f;
            if (m >= 32768.f) q = pow2_scale(m);
            else if (m > 0.f && m < 0.00390625f) q = fmaxf(1.f, fminf(pow2_scale(m), kScaleCap * pow2_inv(sS[ct])));
            if (__ballot(q != 1.f)) {
#pragma unroll
                for (int r = 0; r < DK / 16; ++r) S[ct][r] *= q;
                sS[ct] *= q;
            }
        }
    }
}

// MODE_FUSED: the whole chunk loop per (sequence, head, value block), as
// described at the top.  MODE_PREP: the chunk-operand pass -- phases 1-3 only, for
// PREP_GROUP consecutive chunks (numbered across sequences) of one head per
// workgroup, each chunk's operands stored as its image (no state, no V).
template <typename TIn, int C, int NW, int MODE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(PrefillCfg<TIn, C, NW>::WAVES_PER_EU)))
void kda_prefill_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *initial_state, const int32_t *__restrict__ cu_seqlens,
    int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dv,
    TIn *__restrict__ out, float *final_state, SegArgs seg)
{
    typedef PrefillCfg<TIn, C, NW> P;
    typedef typename P::OpT OpT;
    typedef Mma<OpT> M;
    constexpr bool kIn16 = P::kIn16;
    constexpr int NSUB = P::NSUB, BV = P::BV, NT = P::NT, KB = P::KB, CPT = P::CPT;
    constexpr int SEG = P::SEG, NSEG = P::NSEG, ITEMS = P::ITEMS, GRP = P::GRP, NGRP = P::NGRP;
    constexpr int CPI = P::CPI, IPR = P::IPR;
    constexpr int LDK = P::LDK, LDC = P::LDC, LDK32 = P::LDK32, LDV = P::LDV;
    constexpr float GS = P::GS;

    extern __shared__ __align__(16) unsigned char smem[];
    OpT *sNKp = reinterpret_cast<OpT *>(smem + P::offNKp);
    OpT *sQp = reinterpret_cast<OpT *>(smem + P::offQp);
    OpT *sKc = reinterpret_cast<OpT *>(smem + P::offKc);
    OpT *sKhT = reinterpret_cast<OpT *>(smem + P::offKhT);
    TIn *sV = reinterpret_cast<TIn *>(smem + P::offV);
    TIn *sO = reinterpret_cast<TIn *>(smem + P::offO);
    float *sKr32 = reinterpret_cast<float *>(smem + P::offKr32);
    float *sQr32 = reinterpret_cast<float *>(smem + P::offQr32);
    float *sKD32 = reinterpret_cast<float *>(smem + P::offKD32);
    float *sAd = reinterpret_cast<float *>(smem + P::offAd);
    OpT *sN = reinterpret_cast<OpT *>(smem + P::offN);
    OpT *sT = reinterpret_cast<OpT *>(smem + P::offT);
    OpT *sP = reinterpret_cast<OpT *>(smem + P::offP);
    float *sF = reinterpret_cast<float *>(smem + P::offF);
    float *sH = reinterpret_cast<float *>(smem + P::offH);
    float *sGam = reinterpret_cast<float *>(smem + P::offGam);
    float *sPre = reinterpret_cast<float *>(smem + P::offPre);   // prefix products of group decays
    float *sBeta = reinterpret_cast<float *>(smem + P::offBeta);
    float *sTs = reinterpret_cast<float *>(smem + P::offTs);

    // ---- workgroup -> (work unit, value block); blocks of one unit share an XCD.
    //      A work unit is a (sequence, head) pair, or a (segment, head) pair when
    //      a segment plan is given; summary mode adds DK transition columns.
    constexpr bool kPrep = MODE == MODE_PREP;
    // the fused kernel runs whole sequences; segments run in kda_chain_kernel
    constexpr bool segmented = false;
    constexpr bool summary = false;
    const int wg = blockIdx.x;
    int su = 0, h = 0, n = 0, vb = 0, t_start = 0, t_end = 0, sflags = SEG_FIRST | SEG_LAST;
    int gc_begin = 0, nch = 0;      // chunk-operand pass: first global chunk, chunk count
    if constexpr (kPrep) {
        h = wg % num_heads;
        const int grp = min(max(seg.prep_group, 1), PREP_GROUP);
        gc_begin = (wg / num_heads) * grp;
        const int total_chunks = seg.chunk_off[num_seqs];
        if (gc_begin >= total_chunks) return;
        nch = min(grp, total_chunks - gc_begin);
    } else {
        const int nblk = (summary ? dv + DK : dv) / BV;
        const int xcd = wg & 7, slot = wg >> 3;
        vb = slot % nblk;
        const int64_t unit = (int64_t)(slot / nblk) * 8 + xcd;
        if (unit >= (int64_t)(segmented ? seg.num_segs : num_seqs) * num_heads) return;
        su = (int)(unit / num_heads);
        h = (int)(unit % num_heads);
        n = su;
        if (segmented) {
            n = seg.plan[4 * su];
            t_start = seg.plan[4 * su + 1];
            t_end = seg.plan[4 * su + 2];
            sflags = seg.plan[4 * su + 3];
            if (n < 0 || (summary && (sflags & SEG_LAST))) return;   // unused entry / summary not needed
        } else {
            t_start = cu_seqlens[n];
            t_end = cu_seqlens[n + 1];
        }
        t_start = min(max(t_start, 0), total_tokens);
        t_end = min(max(t_end, t_start), total_tokens);
        nch = (t_end - t_start + C - 1) / C;
    }
    // chunk-operand pass: the token range of each of the workgroup's chunks,
    // found once (thread ci searches chunk_off for chunk gc_begin + ci) and
    // kept in LDS.  Searching inside the chunk loop would put a chain of
    // dependent loads there, and waiting for each of them waits for every
    // memory operation in flight (they complete in order): the prefetched
    // next chunk and the image stores of the previous one.
    __shared__ int32_t prep_rng[2 * PREP_GROUP];
    if constexpr (kPrep) {
        if (threadIdx.x < (unsigned)nch) {
            const int gc = gc_begin + (int)threadIdx.x;
            int lo = 0, hi = num_seqs;                 // chunk_off[lo] <= gc < chunk_off[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (seg.chunk_off[mid] <= gc) lo = mid; else hi = mid;
            }
            const int s0 = min(max(cu_seqlens[lo], 0), total_tokens);
            prep_rng[2 * threadIdx.x + 1] = min(max(cu_seqlens[lo + 1], s0), total_tokens);
            // in range for any valid cu_seqlens; the clamp keeps every load in
            // bounds for any other contents
            prep_rng[2 * threadIdx.x] = min(s0 + (gc - seg.chunk_off[lo]) * C, total_tokens - 1);
        }
        __syncthreads();
    }
    // chunk ci of this workgroup: tokens [c0, min(c0 + C, cend))
    auto chunk_range = [&](int ci, int &c0, int &cend) {
        if constexpr (kPrep) {
            c0 = prep_rng[2 * ci];
            cend = prep_rng[2 * ci + 1];
        } else {
            c0 = t_start + ci * C;
            cend = t_end;
        }
    };
    const int dv0 = vb * BV;
    const bool trans_cols = summary && dv0 >= dv;   // transition columns: V = 0, entering state I

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lj = lane >> 4, lm = lane & 15;
    const int H = num_heads;
    const int64_t rowK = (int64_t)H * DK;      // token stride of q, k, g
    const int64_t rowV = (int64_t)H * dv;      // token stride of v, out
    const int64_t hK = (int64_t)h * DK;

    // slow-prep item of this thread: sub-tile pa, channels pc .. pc + CPT - 1
    const bool prep = tid < P::NPREP;
    const int pa = prep ? tid / (DK / CPT) : 0;
    const int pc = prep ? (tid % (DK / CPT)) * CPT : 0;

    // ---- state slice of this wave: rows 16r + 4*lj + i, column dv0 + 16*wave + lm
    f32x4 Sarr[1][DK / 16];
    f32x4 (&S)[DK / 16] = Sarr[0];
    const int col = dv0 + 16 * wave + lm;
    const int64_t sbase = ((int64_t)n * num_heads + h) * DK * dv;   // this (sequence, head) in init/final
    const float *S_in = nullptr;
    int64_t S_in_base = 0;
    if (summary) {
        S_in = nullptr;                                   // zero (value columns) or identity
    } else if (segmented) {
        // every segment, a first one included, enters from seg_init: the
        // initial state was copied there before this pass, so a last segment
        // may overwrite it (final_state == initial_state) while others run
        S_in = seg.seg_init;
        S_in_base = (seg_init_entry(seg, su, n, t_start, cu_seqlens, total_tokens) * num_heads + h) * DK * dv;
    } else if (initial_state) {
        S_in = initial_state;
        S_in_base = sbase;
    }
    if (S_in) {
#pragma unroll
        for (int r = 0; r < DK / 16; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[r][i] = S_in[S_in_base + (int64_t)(16 * r + 4 * lj + i) * dv + col];
    } else {
#pragma unroll
        for (int r = 0; r < DK / 16; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[r][i] = (trans_cols && 16 * r + 4 * lj + i == col - dv) ? 1.f : 0.f;
    }
    // the state is carried scaled per column by a power of two (see chain_chunk)
    float sSarr[1] = {1.f};
    float &sS = sSarr[0];
    if (kIn16) {
        float m = 0.f;
#pragma unroll
        for (int r = 0; r < DK / 16; ++r) m = absmax_acc(m, S[r]);
        sS = fminf(pow2_scale(colmax(m)), kScaleCap);
#pragma unroll
        for (int r = 0; r < DK / 16; ++r) S[r] *= sS;
    }

    // ---- raw chunk data staged in registers, loaded one chunk ahead: item it
    //      of this thread is segment (tid + it NT) / 64, channels 2 ((tid + it NT) % 64) + {0, 1}.
    //      Rows past the end of the sequence read the last valid row (in bounds)
    //      and are masked where they are used, so every load is unconditional.
    constexpr int VEC = 16 / (int)sizeof(TIn);            // elements per 16-byte vector
    constexpr int VPR = BV / VEC;                         // vectors per token row
    constexpr int VITEMS = (C * VPR + NT - 1) / NT;
    typedef typename Quad<TIn>::type QuadT;
    f32x4 rg[ITEMS][SEG];
    QuadT rk[ITEMS][SEG], rq[ITEMS][SEG];
    f32x4 rv[VITEMS];
    float rb = 0.f;
    auto load_chunk = [&](int cc0, int cend) {
        const int LL = max(1, min(C, cend - cc0));
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = min(tid + it * NT, NSEG * IPR - 1), sg = item / IPR, c = CPI * (item % IPR);
#pragma unroll
            for (int rr = 0; rr < SEG; ++rr) {
                const int rc = min(sg * SEG + rr, LL - 1);
                const int64_t off = (int64_t)(cc0 + rc) * rowK + hK + c;
                rg[it][rr] = *reinterpret_cast<const f32x4 *>(g + off);
                rk[it][rr] = *reinterpret_cast<const QuadT *>(k + off);
                rq[it][rr] = *reinterpret_cast<const QuadT *>(q + off);
            }
        }
#pragma unroll
        for (int it = 0; it < (kPrep ? 0 : VITEMS); ++it) {
            const int e = tid + it * NT;
            if (e < C * VPR) {
                const int rc = min(e / VPR, LL - 1), cv = (e % VPR) * VEC;
                rv[it] = trans_cols ? zero4()
                                    : *reinterpret_cast<const f32x4 *>(v + (int64_t)(cc0 + rc) * rowV + (int64_t)h * dv + dv0 + cv);
            }
        }
        rb = beta[(int64_t)(cc0 + min(tid, LL - 1)) * H + h];   // used by tid < C; unconditional, as above
    };
    if (kPrep || nch > 0) {   // (the chunk-operand pass has nch >= 1: no branch around its loads)
        int a0, a1;
        chunk_range(0, a0, a1);
        load_chunk(a0, a1);
    }

    // product of the group decays over groups [g0, g1) of channel c, in order
    auto grp_prod = [&](int g0, int g1, int c) {
        float p = 1.f;
        for (int s = g0; s < g1; ++s) p *= sF[s * DK + c];
        return p;
    };
    constexpr int GPS = SUB / GRP;                        // groups per sub-tile

    // chunk-operand pass: LDS byte offsets of this thread's image vectors (fixed)
    typedef ChunkImage<TIn, C> Img;
    constexpr int SITEMS = kPrep ? (Img::NVEC + NT - 1) / NT : 1;
    uint32_t img_off[SITEMS];
    if constexpr (kPrep) {
        const typename Img::Offs o = {(uint32_t)P::offNKp, (uint32_t)P::offQp, (uint32_t)P::offKhT,
                                      (uint32_t)P::offT, (uint32_t)P::offP, (uint32_t)P::offGam,
                                      (uint32_t)P::offBeta, (uint32_t)P::offTs};
#pragma unroll
        for (int it = 0; it < SITEMS; ++it) img_off[it] = Img::lds_off(min(tid + it * NT, Img::NVEC - 1), o);
        // One placeholder store per image item after the first chunk's loads,
        // so that the loop is entered as it is re-entered from its end (the
        // chunk's loads followed by SITEMS stores): the compiler merges the two
        // paths at the loop head and, were they to differ, would count as if
        // there were no stores after the loads, and wait for the previous
        // chunk's image stores before each use of the prefetched data.  The
        // placeholders go to the last image slot of this head, which valid
        // input never uses (there are more slots than chunks); every
        // workgroup of the head writes the same zeros there, so the lines
        // stay in L2.  (nch >= 1 here: a workgroup without chunks has returned)
        f32x4 *junk = seg.img + ((int64_t)(seg.img_slots - 1) * num_heads + h) * Img::NVEC;
#pragma unroll
        for (int it = 0; it < SITEMS; ++it) junk[min(tid + it * NT, Img::NVEC - 1)] = zero4();
    }
    for (int ci = 0; ci < nch; ++ci) {
        int c0, cend;
        chunk_range(ci, c0, cend);
        const int L = min(C, cend - c0);         // valid tokens in this chunk
        __syncthreads();                          // previous chunk done with all LDS

        // ---- 1a. group gate sums -> F = exp(sum); beta
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = tid + it * NT, sg = item / IPR, c = CPI * (item % IPR);
            if (item < NSEG * IPR) {
#pragma unroll
                for (int gi = 0; gi < SEG / GRP; ++gi) {
                    f32x4 sum = zero4();
#pragma unroll
                    for (int rr = gi * GRP; rr < (gi + 1) * GRP; ++rr) {
                        const bool ok = sg * SEG + rr < L;
#pragma unroll
                        for (int x = 0; x < CPI; ++x) sum[x] += ok ? rg[it][rr][x] : 0.f;
                    }
                    const int G = (sg * SEG) / GRP + gi;
                    f32x4 f;
#pragma unroll
                    for (int x = 0; x < CPI; ++x) f[x] = __expf(sum[x]);
                    *reinterpret_cast<f32x4 *>(sF + G * DK + c) = f;
                }
            }
        }
        if (tid < C) sBeta[tid] = tid < L ? rb : 0.f;
        __syncthreads();

        // ---- 1b. gamma = prod of all group decays; decay-span test; sub-tile
        //          tables H(a,b) for the strong-decay Gram
        int strong = 0;
        for (int c = tid; c < DK; c += NT) {
            float gm = 1.f;                         // same order as grp_prod(0, G, c)
            sPre[c] = gm;
            for (int G = 0; G < NGRP; ++G) {
                gm *= sF[G * DK + c];
                sPre[(G + 1) * DK + c] = gm;
            }
            sGam[c] = gm;
            strong |= gm < __expf(-P::SPAN_CHUNK);
        }
        const bool slow = __syncthreads_or(strong);
        if (slow) {
            for (int e = tid; e < P::NPAIR * DK; e += NT) {
                const int p = e / DK, c = e % DK;
                int a, b;
                pair_of(p, a, b);
                sH[p * DK + c] = (b == a) ? 1.f / grp_prod(a * GPS, (a + 1) * GPS, c)
                                          : grp_prod((b + 1) * GPS, a * GPS, c);
            }
        }

        // ---- 1c. decayed operands
        // fast: from the staged registers, chunk-start reference R_r = e^Gamma_r,
        //       written once for both the Gram and the chain
        // FULL: every row of the chunk is a token (no masking needed)
        auto prep_fast = [&](auto full_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            typedef OpT V4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int it = 0; it < ITEMS; ++it) {
                const int item = tid + it * NT, sg = item / IPR, c = CPI * (item % IPR);
                if (item >= NSEG * IPR) continue;
                const int G0 = (sg * SEG) / GRP;
                const int pc4 = kperm<OpT>(c);              // channels c .. c + 3 stay contiguous
                f32x4 pre = *reinterpret_cast<const f32x4 *>(sPre + G0 * DK + c);   // prefix over earlier groups
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(sGam + c);        // all groups
                OpT kh[CPI][SEG];
                f32x4 R;
#pragma unroll
                for (int rr = 0; rr < SEG; ++rr) {
                    const int r = sg * SEG + rr;
                    const bool ok = FULL || r < L;
                    if (rr % GRP == 0) {
                        if (rr > 0) pre = *reinterpret_cast<const f32x4 *>(sPre + (G0 + rr / GRP) * DK + c);
                        R = f32x4{1.f, 1.f, 1.f, 1.f};
                    }
                    V4 nk, qq, kc;
#pragma unroll
                    for (int x = 0; x < CPI; ++x) {
                        const float kx = ok ? to_f(rk[it][rr][x]) : 0.f, qx = ok ? to_f(rq[it][rr][x]) : 0.f;
                        R[x] *= ok ? __expf(rg[it][rr][x]) : 1.f;     // decay inside the group
                        const float e = pre[x] * R[x];                 // e^Gamma_r
                        const float ie = __builtin_amdgcn_rcpf(e);
                        nk[x] = from_f<OpT>(-GS * kx * e);
                        qq[x] = from_f<OpT>(GS * qx * e);
                        kc[x] = from_f<OpT>(kx * ie * (1.f / GS));
                        kh[x][rr] = from_f<OpT>(GS * kx * (gm[x] * ie));
                    }
                    *reinterpret_cast<V4 *>(sNKp + r * LDK + pc4) = nk;
                    *reinterpret_cast<V4 *>(sQp + r * LDK + pc4) = qq;
                    *reinterpret_cast<V4 *>(sKc + r * LDK + pc4) = kc;
                }
                // K^ transposed: SEG consecutive tokens of channels c .. c + 3
#pragma unroll
                for (int rr = 0; rr < SEG; rr += 4) {
                    const int pt = kperm<OpT>(sg * SEG + rr);   // 4 tokens stay contiguous
#pragma unroll
                    for (int x = 0; x < CPI; ++x) {
                        V4 w;
#pragma unroll
                        for (int y = 0; y < 4; ++y) w[y] = kh[x][rr + y];
                        *reinterpret_cast<V4 *>(sKhT + (c + x) * LDC + pt) = w;
                    }
                }
            }
        };
        if (slow)
            prep_slow<TIn, C, NW>(true, q, k, g, c0, L, rowK, hK, tid, sF, sKr32, sQr32, sKD32, sNKp, sQp, sKhT);
        else if (L == C)
            prep_fast(std::true_type());
        else
            prep_fast(std::false_type());
        // chunk-operand pass: the staged registers are free once the decayed
        // operands are written, so the next chunk's loads go out here and
        // stay in flight through the Gram, the inverse and the image store
        // (the fused kernel still needs its value registers until phase 3)
        if constexpr (kPrep) {
            int n0, n1;
            chunk_range(min(ci + 1, nch - 1), n0, n1);
            if (ci + 1 >= nch) n1 = n0 + 1;     // nothing left: every lane reads one (cached) row
            load_chunk(n0, n1);
        }
        __syncthreads();

        // ---- 2. Gram tiles
        if (slow)
            gram_tiles<float, OpT, C, NW>(sKr32, sQr32, sKD32, LDK32, sH, 1.f, sBeta, sAd, sN, sP, LDC,
                                          wave, lj, lm);
        else   // rows hold -GS K+ and GS Q+, columns K e^-Gamma / GS
            gram_tiles<OpT, OpT, C, NW>(sNKp, sQp, sKc, LDK, nullptr, -1.f, sBeta, sAd, sN, sP, LDC,
                                        wave, lj, lm);
        __syncthreads();

        // ---- 3. chain operands after a slow Gram; value tile; next chunk's
        //         loads (they overlap the rest of this chunk); diagonal blocks of
        //         (I + N)^-1 by forward substitution, lane = column
        if (slow)
            prep_slow<TIn, C, NW>(false, q, k, g, c0, L, rowK, hK, tid, sF, sKr32, sQr32, sKD32, sNKp, sQp, sKhT);
#pragma unroll
        for (int it = 0; it < (kPrep ? 0 : VITEMS); ++it) {
            const int e = tid + it * NT;
            if (e < C * VPR) {
                const int r = e / VPR, cv = (e % VPR) * VEC;
                *reinterpret_cast<f32x4 *>(sV + r * LDV + cv) = r < L ? rv[it] : zero4();
            }
        }
        // unconditional (the last chunk re-reads itself): a conditional load
        // would make the compiler wait for it right away
        if constexpr (!kPrep) {
            int n0, n1;
            chunk_range(min(ci + 1, nch - 1), n0, n1);
            load_chunk(n0, n1);
        }
        if (tid < NSUB * SUB) {
            const int a = tid / SUB, nc = tid % SUB;
            const float *NT = sAd + a * SUB * P::LDAD;     // NT[s][r] = N[r][s]
            // Forward substitution, lane = column.  The 4-aligned tails of the
            // columns below the diagonal are read in batches ahead of the
            // steps that use them: read one step at a time, every read's
            // latency would sit on the dependent chain.
            float x[SUB];
#pragma unroll
            for (int r = 0; r < SUB; ++r) x[r] = (r == nc) ? 1.f : 0.f;
            auto solve = [&](auto s0_tag, auto s1_tag) {
                constexpr int S0 = decltype(s0_tag)::value, S1 = decltype(s1_tag)::value;
                f32x4 tv[tail_vecs(S0, S1)];
                int v = 0;
#pragma unroll
                for (int s = S0; s < S1; ++s)
#pragma unroll
                    for (int q4 = (s + 1) & ~3; q4 < SUB; q4 += 4)
                        tv[v++] = *reinterpret_cast<const f32x4 *>(NT + s * P::LDAD + q4);
                v = 0;
#pragma unroll
                for (int s = S0; s < S1; ++s)
#pragma unroll
                    for (int q4 = (s + 1) & ~3; q4 < SUB; q4 += 4) {
                        const f32x4 t = tv[v++];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (q4 + e > s) x[q4 + e] -= t[e] * x[s];
                    }
            };
            solve(std::integral_constant<int, 0>(), std::integral_constant<int, 3>());
            solve(std::integral_constant<int, 3>(), std::integral_constant<int, 7>());
            solve(std::integral_constant<int, 7>(), std::integral_constant<int, 11>());
            solve(std::integral_constant<int, 11>(), std::integral_constant<int, SUB - 1>());
            // fp16 range: scale the block down by a power of two if it exceeds 2^14
            float sc = 1.f;
            if (kIn16) {
                float m = 0.f;
#pragma unroll
                for (int r = 0; r < SUB; ++r) m = fmaxf(m, fabsf(x[r]));
                m = rowmax16(m);                         // the 16 lanes of block a
                if (m > 16384.f) sc = pow2_scale(m);
            }
            if (nc == 0) sTs[a * NSUB + a] = pow2_inv(sc);
#pragma unroll
            for (int r = 0; r < SUB; ++r) sT[(a * SUB + r) * LDC + a * SUB + nc] = from_f<OpT>(x[r] * sc);
        }
        __syncthreads();

        // ---- 3b. off-diagonal blocks: T_ab = -T_aa sum_{b<=s<a} N_as T_sb, by distance a-b
#pragma unroll
        for (int d = 1; d < NSUB; ++d) {
            for (int b = wave; b + d < NSUB; b += NW) {
                const int a = b + d;
                f32x4 y = zero4();
                const OpT *rowN = sN + (a * SUB + lm) * LDC;
                for (int s = b; s < a; ++s) {
                    const f32x4 t = M::mma16(M::load16(rowN, s * SUB, lj),
                                             load16_col(sT + (s * SUB) * LDC + b * SUB, LDC, lj, lm), zero4());
                    y += t * sTs[s * NSUB + b];
                }
                float sy = 1.f;
                if (kIn16) sy = pow2_scale(colmax(absmax4(y)));
                f32x4 t = M::mma16(M::load16(sT + (a * SUB + lm) * LDC, a * SUB, lj), M::from_acc16(y, sy), zero4());
                t *= -(sTs[a * NSUB + a] * pow2_inv(sy));
                float sc = 1.f;
                if (kIn16) {
                    const float m = wavemax(absmax4(t));
                    if (m > 16384.f) sc = pow2_scale(m);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sT[(a * SUB + 4 * lj + i) * LDC + b * SUB + lm] = from_f<OpT>(t[i] * sc);
                if (lane == 0) sTs[a * NSUB + b] = pow2_inv(sc);
            }
            __syncthreads();
        }

        if constexpr (kPrep) {
            // ---- chunk-operand image of (chunk, head) -> global
            f32x4 *dst = seg.img + ((int64_t)(gc_begin + ci) * num_heads + h) * Img::NVEC;
            // all LDS reads first, then the stores; surplus items repeat the last
            // vector (same value, same place) so that every store is issued
            f32x4 tv[SITEMS];
#pragma unroll
            for (int it = 0; it < SITEMS; ++it) tv[it] = *reinterpret_cast<const f32x4 *>(smem + img_off[it]);
#pragma unroll
            for (int it = 0; it < SITEMS; ++it) dst[min(tid + it * NT, Img::NVEC - 1)] = tv[it];
            continue;
        }
        // ---- 4. state-dependent chain (this wave's 16 columns)
        chain_chunk<TIn, C, LDV, LDV, false>(Sarr, sSarr, sNKp, sQp, sKhT, sT, sP, sTs, sGam, sBeta, sV, 16 * wave + lm, sO,
                                             16 * wave + lm, lj, lm);
        __syncthreads();

        // ---- 5. output tile -> global (valid tokens only)
        for (int e = tid; e < (summary || !out ? 0 : C * VPR); e += NT) {   // out: NULL only when snapshotting
            const int r = e / VPR, cv = (e % VPR) * VEC;
            if (r < L)
                *reinterpret_cast<f32x4 *>(out + (int64_t)(c0 + r) * rowV + (int64_t)h * dv + dv0 + cv) =
                    *reinterpret_cast<const f32x4 *>(sO + r * LDV + cv);
        }
        // ---- state snapshot when this chunk ends (snap_every)-aligned tokens
        //      into the sequence (prefix caching)
        //      Packed form (chunk_off given): the state at the start of every
        //      chunk but a sequence's first, at its global chunk index.
        if (MODE == MODE_SNAP && L == C &&
            (seg.chunk_off ? ci + 1 < nch : ((ci + 1) * C) % seg.snap_every == 0)) {
            const int j = seg.chunk_off ? seg.chunk_off[n] + ci + 1 : (ci + 1) * C / seg.snap_every - 1;
            if (seg.chunk_off || j < seg.max_snaps) {
                float *dst = seg.snap + ((seg.chunk_off ? (int64_t)j : (int64_t)n * seg.max_snaps + j) * num_heads + h) *
                                            DK * dv;
#pragma unroll
                for (int r = 0; r < DK / 16; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dst[(int64_t)(16 * r + 4 * lj + i) * dv + col] = S[r][i] * pow2_inv(sS);
            }
        }
    }

    if (summary) {
        // segment summary: [S_end from zero | segment transition], row stride dv + DK
        float *dst = seg.seg_out + ((int64_t)su * num_heads + h) * DK * (dv + DK);
#pragma unroll
        for (int r = 0; r < DK / 16; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(int64_t)(16 * r + 4 * lj + i) * (dv + DK) + col] = S[r][i] * pow2_inv(sS);
    } else if (final_state && (sflags & SEG_LAST)) {
#pragma unroll
        for (int r = 0; r < DK / 16; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                final_state[sbase + (int64_t)(16 * r + 4 * lj + i) * dv + col] = S[r][i] * pow2_inv(sS);
    }
}

// ------------------------------------------------------------------ launch
template <typename TIn, int C, int NW, int MODE>
static hipError_t launch_prefill_t(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *init, const int32_t *cu,
                                   int32_t N, int32_t T_tot, int32_t H, int32_t dv, void *out,
                                   float *fin, SegArgs seg, hipStream_t stream)
{
    typedef PrefillCfg<TIn, C, NW> P;
    auto kern = kda_prefill_kernel<TIn, C, NW, MODE>;
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(kern), (int)P::bytes, lds_set)) return e;
    const int64_t units = (int64_t)N * H;
    const int nblk = dv / P::BV;
    const int64_t groups = (units + 7) / 8;
    const int64_t grid = groups * 8 * nblk;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(P::NT), P::bytes, stream,
                       static_cast<const TIn *>(q), static_cast<const TIn *>(k), static_cast<const TIn *>(v),
                       g, beta, init, cu, N, T_tot, H, dv, static_cast<TIn *>(out), fin, seg);
    return hipGetLastError();
}


// ------------------------------------------------------------ state chain
// The state-dependent pass over chunk-operand images: one workgroup per
// (unit, block of BV value columns) as in the fused kernel, walking the unit's
// chunks in order.  Per chunk: the next chunk's image and value tile are
// loaded into registers, the chain runs on the current LDS buffer, each wave
// stores its own output columns, and the registers are written to the LDS.
// Double-buffered (SB = false): one barrier per chunk, the registers go to the
// other buffer.  Single-buffered (SB = true): a second barrier before the
// registers overwrite the one buffer; half the LDS, so that two workgroups
// share a compute unit and one runs while the other waits.
template <typename TIn, int C, int NW, int NCT, bool SB = false>
struct ChainCfg {
    typedef PrefillCfg<TIn, C, NW> P;
    typedef typename P::OpT OpT;
    typedef ChunkImage<TIn, C> Img;
    static constexpr int NT = 64 * NW, BV = 16 * NW * NCT, NSUB = C / SUB;   // NCT 16-column tiles per wave
    static constexpr int LDK = P::LDK, LDC = P::LDC, LDV = BV + 16 / (int)sizeof(TIn);
    static constexpr uint32_t offNKp = 0;
    static constexpr uint32_t offQp = offNKp + sizeof(OpT) * C * LDK;
    static constexpr uint32_t offKhT = offQp + sizeof(OpT) * C * LDK;
    static constexpr uint32_t offT = offKhT + sizeof(OpT) * DK * LDC;
    static constexpr uint32_t offP = offT + sizeof(OpT) * C * LDC;
    static constexpr uint32_t offGam = offP + sizeof(OpT) * C * LDC;
    static constexpr uint32_t offBeta = offGam + sizeof(float) * DK;
    static constexpr uint32_t offTs = offBeta + sizeof(float) * C;
    static constexpr uint32_t offV = offTs + (sizeof(float) * NSUB * NSUB + 15) / 16 * 16;
    static constexpr uint32_t BUF = (offV + sizeof(TIn) * C * LDV + 15) / 16 * 16;   // one chunk buffer
    static constexpr uint32_t offO = (SB ? 1 : 2) * BUF;                       // [NW][C][16 NCT] outputs
    static constexpr uint32_t bytes = offO + sizeof(TIn) * NW * C * 16 * NCT;
    static_assert(bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
    static constexpr int WG_PER_CU = (2 * bytes <= 160 * 1024) ? 2 : 1;
    static constexpr int WAVES_PER_EU = (WG_PER_CU * NW) / 4 >= 2 ? 2 : 1;
    static constexpr int IITEMS = (Img::NVEC + NT - 1) / NT;        // image vectors per thread (outputs)
    static constexpr int IITEMS_SUM = (Img::NVEC_SUM + NT - 1) / NT; // (summaries: no Q+, P)
    static constexpr int VEC = 16 / (int)sizeof(TIn);               // elements per 16-byte vector
    static constexpr int VPR = BV / VEC;                            // vectors per value-tile row
    static constexpr int VITEMS = (C * VPR + NT - 1) / NT;
    static constexpr int OVEC = C * 16 * NCT / VEC;                 // vectors of one wave's output tile
};

// SNAP (outputs only): also store the state after every chunk that is not its
// sequence's last, as the state at the start of the next chunk, at that
// chunk's global index in seg.snap ([chunks][H][DK][dv]); out may be NULL.
template <typename TIn, int C, int NW, int NCT, bool SUMMARY, bool SB, bool SNAP = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(ChainCfg<TIn, C, NW, NCT, SB>::WAVES_PER_EU)))
void kda_chain_kernel(const TIn *v, const float *initial_state, const int32_t *__restrict__ cu_seqlens,
                      int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dv,
                      TIn *__restrict__ out, float *final_state, SegArgs seg)
{
    typedef ChainCfg<TIn, C, NW, NCT, SB> Q;
    typedef typename Q::OpT OpT;
    typedef typename Q::Img Img;
    constexpr int NT = Q::NT, BV = Q::BV, LDV = Q::LDV, VEC = Q::VEC, VPR = Q::VPR;
    extern __shared__ __align__(16) unsigned char smem[];

    // ---- workgroup -> (unit, value block): as in the fused kernel
    const bool segmented = seg.plan != nullptr;
    constexpr bool summary = SUMMARY;
    const int nblk = (summary ? dv + DK : dv) / BV;
    const int wg = blockIdx.x;
    const int xcd = wg & 7, slot = wg >> 3;
    const int vb = slot % nblk;
    const int64_t unit = (int64_t)(slot / nblk) * 8 + xcd;
    if (unit >= (int64_t)(segmented ? seg.num_segs : num_seqs) * num_heads) return;
    int su = (int)(unit / num_heads);
    const int h = (int)(unit % num_heads);
    int n = su, t_start, t_end, sflags = SEG_FIRST | SEG_LAST;
    if (segmented) {
        if (seg.sched) su = min(max(seg.sched[su], 0), seg.num_segs - 1);
        n = seg.plan[4 * su];
        t_start = seg.plan[4 * su + 1];
        t_end = seg.plan[4 * su + 2];
        sflags = seg.plan[4 * su + 3];
        if (n < 0 || (summary && (sflags & SEG_LAST))) return;
    } else {
        t_start = cu_seqlens[n];
        t_end = cu_seqlens[n + 1];
    }
    const int seq_start = min(max(cu_seqlens[n], 0), total_tokens);
    t_start = min(max(t_start, 0), total_tokens);
    t_end = min(max(t_end, t_start), total_tokens);
    const int64_t gc0 = seg.chunk_off[n] + (t_start - seq_start) / C;   // first global chunk
    // the images cover chunks [0, chunk_off[N]); the bound only binds when
    // cu_seqlens is not non-decreasing (result unspecified, memory safe)
    const int nch = (int)max((int64_t)0, min((int64_t)(t_end - t_start + C - 1) / C,
                                             (int64_t)seg.chunk_off[num_seqs] - gc0));
    const int dv0 = vb * BV;                 // summary blocks may span value and transition columns

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lj = lane >> 4, lm = lane & 15;
    const int H = num_heads;
    const int64_t rowV = (int64_t)H * dv;

    // ---- entering state: tile ct of this wave is column dv0 + 16 (NCT wave + ct) + lm
    f32x4 S[NCT][DK / 16];
    float sS[NCT];
    int colc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) colc[ct] = dv0 + 16 * (NCT * wave + ct) + lm;
    const int64_t sbase = ((int64_t)n * num_heads + h) * DK * dv;
    const float *S_in = nullptr;
    int64_t S_in_base = 0;
    if (summary) {
        S_in = nullptr;
    } else if (segmented) {
        S_in = seg.seg_init;
        S_in_base = (seg_init_entry(seg, su, n, t_start, cu_seqlens, total_tokens) * num_heads + h) * DK * dv;
    } else if (initial_state) {
        S_in = initial_state;
        S_in_base = sbase;
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int col = colc[ct];
        if (S_in) {
#pragma unroll
            for (int r = 0; r < DK / 16; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[ct][r][i] = S_in[S_in_base + (int64_t)(16 * r + 4 * lj + i) * dv + col];
        } else {   // zero; a summary's transition columns start from the identity
#pragma unroll
            for (int r = 0; r < DK / 16; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[ct][r][i] = (summary && 16 * r + 4 * lj + i == col - dv) ? 1.f : 0.f;
        }
        // the state is carried scaled per column by a power of two (see chain_chunk)
        sS[ct] = 1.f;
        if (Q::P::kIn16) {
            float m = 0.f;
#pragma unroll
            for (int r = 0; r < DK / 16; ++r) m = absmax_acc(m, S[ct][r]);
            sS[ct] = fminf(pow2_scale(colmax(m)), kScaleCap);
#pragma unroll
            for (int r = 0; r < DK / 16; ++r) S[ct][r] *= sS[ct];
        }
    }

    // ---- chunk staging: image + value tile of chunk ci in registers
    constexpr int IIT = SUMMARY ? Q::IITEMS_SUM : Q::IITEMS;       // image vectors this pass reads
    constexpr int NV = SUMMARY ? Img::NVEC_SUM : Img::NVEC;
    f32x4 ri[IIT], rv[Q::VITEMS], ri2[IIT], rv2[Q::VITEMS];
    auto load_to = [&](int ci, f32x4 (&ri)[IIT], f32x4 (&rv)[Q::VITEMS]) {
        const f32x4 *src = seg.img + ((gc0 + ci) * H + h) * Img::NVEC;
#pragma unroll
        for (int it = 0; it < IIT; ++it) ri[it] = src[min(tid + it * NT, NV - 1)];
        const int c0 = t_start + ci * C, LL = min(C, t_end - c0);
#pragma unroll
        for (int it = 0; it < Q::VITEMS; ++it) {
            const int e = min(tid + it * NT, C * VPR - 1);
            const int rc = min(e / VPR, LL - 1), cv = (e % VPR) * VEC;
            // transition columns (V = 0) read the row's last value vector,
            // zeroed when staged: with no branch around the load the compiler
            // counts the loads in flight exactly, and does not wait for newer
            // ones (a zero chosen here would become such a branch)
            rv[it] = *reinterpret_cast<const f32x4 *>(v + (int64_t)(c0 + rc) * rowV + (int64_t)h * dv +
                                                      min(dv0 + cv, dv - VEC));
        }
    };
    auto load = [&](int ci) { load_to(ci, ri, rv); };
    const typename Img::Offs offs = {Q::offNKp, Q::offQp, Q::offKhT, Q::offT, Q::offP, Q::offGam, Q::offBeta, Q::offTs};
    uint32_t stage_off[IIT];                              // LDS byte offsets of this thread's image vectors
#pragma unroll
    for (int it = 0; it < IIT; ++it) stage_off[it] = Img::lds_off(min(tid + it * NT, NV - 1), offs);
    // Every staged register is written on every path (surplus items repeat
    // the last vector, same value to the same place): a conditional consumer
    // would leave the loads pending at the loop head for the compiler, which
    // then waits there for all older memory operations, output stores included.
    auto stage_from = [&](int ci, int b, const f32x4 (&ri)[IIT], const f32x4 (&rv)[Q::VITEMS]) {
        unsigned char *base = smem + b * Q::BUF;
#pragma unroll
        for (int it = 0; it < IIT; ++it) *reinterpret_cast<f32x4 *>(base + stage_off[it]) = ri[it];
        TIn *sV = reinterpret_cast<TIn *>(base + Q::offV);
        const int LL = min(C, t_end - (t_start + ci * C));
#pragma unroll
        for (int it = 0; it < Q::VITEMS; ++it) {
            const int e = min(tid + it * NT, C * VPR - 1);
            const int r = e / VPR, cv = (e % VPR) * VEC;
            *reinterpret_cast<f32x4 *>(sV + r * LDV + cv) = r < LL && dv0 + cv < dv ? rv[it] : zero4();
        }
    };
    auto stage = [&](int ci, int b) { stage_from(ci, b, ri, rv); };
    if constexpr (SUMMARY && !SB) {
        // summaries: the operands are loaded two chunks ahead, into register
        // sets A (ri, rv) and B (ri2, rv2) in turn, so that a load has two
        // chunks' work to arrive; the loop takes chunks in pairs to keep the
        // sets apart, and a compiler barrier after each load keeps it from
        // being moved next to its use
        auto run = [&](int ci) {
            const unsigned char *base = smem + (ci & 1) * Q::BUF;
            chain_chunk<TIn, C, LDV, 16 * NCT, SUMMARY, NCT>(
                S, sS, reinterpret_cast<const OpT *>(base + Q::offNKp), reinterpret_cast<const OpT *>(base + Q::offQp),
                reinterpret_cast<const OpT *>(base + Q::offKhT), reinterpret_cast<const OpT *>(base + Q::offT),
                reinterpret_cast<const OpT *>(base + Q::offP), reinterpret_cast<const float *>(base + Q::offTs),
                reinterpret_cast<const float *>(base + Q::offGam), reinterpret_cast<const float *>(base + Q::offBeta),
                reinterpret_cast<const TIn *>(base + Q::offV), 16 * NCT * wave + lm, nullptr, lm, lj, lm);
        };
        if (nch > 0) {
            load_to(0, ri, rv);
            stage_from(0, 0, ri, rv);
            load_to(min(1, nch - 1), ri, rv);
        }
        int ci = 0;
        for (; ci + 2 <= nch; ci += 2) {
            __syncthreads();
            load_to(min(ci + 2, nch - 1), ri2, rv2);
            asm volatile("" ::: "memory");
            run(ci);
            stage_from(min(ci + 1, nch - 1), (ci + 1) & 1, ri, rv);
            __syncthreads();
            load_to(min(ci + 3, nch - 1), ri, rv);
            asm volatile("" ::: "memory");
            run(ci + 1);
            stage_from(min(ci + 2, nch - 1), ci & 1, ri2, rv2);
        }
        if (ci < nch) {
            __syncthreads();
            run(ci);
        }
    } else {
    if (nch > 0) {
        load(0);
        stage(0, 0);
    }
    TIn *sOw = reinterpret_cast<TIn *>(smem + Q::offO) + wave * C * 16 * NCT;   // this wave's output tile
    for (int ci = 0; ci < nch; ++ci) {
        __syncthreads();                          // chunk ci staged; (double buffer) ci - 1 done with the other
        load(min(ci + 1, nch - 1));               // unconditional, see the fused kernel
        const unsigned char *base = smem + (SB ? 0 : (ci & 1) * Q::BUF);
        chain_chunk<TIn, C, LDV, 16 * NCT, SUMMARY, NCT>(
            S, sS, reinterpret_cast<const OpT *>(base + Q::offNKp), reinterpret_cast<const OpT *>(base + Q::offQp),
            reinterpret_cast<const OpT *>(base + Q::offKhT), reinterpret_cast<const OpT *>(base + Q::offT),
            reinterpret_cast<const OpT *>(base + Q::offP), reinterpret_cast<const float *>(base + Q::offTs),
            reinterpret_cast<const float *>(base + Q::offGam), reinterpret_cast<const float *>(base + Q::offBeta),
            reinterpret_cast<const TIn *>(base + Q::offV), 16 * NCT * wave + lm, sOw, lm, lj, lm);
        if (!SUMMARY && (!SNAP || out)) {
            // this wave's 16 output columns: rows of 16 * sizeof(TIn) bytes, one
            // 16-byte vector per lane and step (LDS is in order within a wave).
            // Every lane stores on every path -- rows past the end of the
            // sequence rewrite the last valid row with its own value -- so that
            // the compiler can count the store and need not wait for it later.
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const int c0 = t_start + ci * C, L = min(C, t_end - c0);
            constexpr int VPW = 16 * NCT / VEC;                        // vectors per row of the tile
#pragma unroll
            for (int e = lane; e < Q::OVEC; e += 64) {
                const int r = min(e / VPW, L - 1), cv = (e % VPW) * VEC;
                *reinterpret_cast<f32x4 *>(out + (int64_t)(c0 + r) * rowV + (int64_t)h * dv + dv0 + 16 * NCT * wave + cv) =
                    *reinterpret_cast<const f32x4 *>(sOw + r * 16 * NCT + cv);
            }
            __asm__ volatile("" ::: "memory");
        }
        if constexpr (SNAP) {
            const int64_t gc = gc0 + ci + 1;            // the sequence's next chunk
            if (gc < (int64_t)seg.chunk_off[n + 1]) {
                float *dst = seg.snap + (gc * num_heads + h) * DK * dv;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const float inv = pow2_inv(sS[ct]);
#pragma unroll
                    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            dst[(int64_t)(16 * r + 4 * lj + i) * dv + colc[ct]] = S[ct][r][i] * inv;
                }
            }
        }
        if constexpr (SB) __syncthreads();       // every wave is done with the buffer
        stage(min(ci + 1, nch - 1), SB ? 0 : (ci + 1) & 1);
    }
    }

#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int col = colc[ct];
        const float inv = pow2_inv(sS[ct]);
        if (summary) {
            float *dst = seg.seg_out + ((int64_t)su * num_heads + h) * DK * (dv + DK);
#pragma unroll
            for (int r = 0; r < DK / 16; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(int64_t)(16 * r + 4 * lj + i) * (dv + DK) + col] = S[ct][r][i] * inv;
        } else if (final_state && (sflags & SEG_LAST)) {
#pragma unroll
            for (int r = 0; r < DK / 16; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    final_state[sbase + (int64_t)(16 * r + 4 * lj + i) * dv + col] = S[ct][r][i] * inv;
        }
    }
}

template <typename TIn, int C>
static hipError_t launch_prep_t(const void *q, const void *k, const float *g, const float *beta,
                                const int32_t *cu, int32_t N, int32_t T_tot, int32_t H, int64_t max_chunks,
                                SegArgs seg, hipStream_t stream)
{
    typedef PrefillCfg<TIn, C, 4> P;
    auto kern = kda_prefill_kernel<TIn, C, 4, MODE_PREP>;
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(kern), (int)P::bytes, lds_set)) return e;
    // fewer chunks per workgroup when there are few: every compute unit
    // gets work, and a workgroup's walk is short
    const int64_t want = (max_chunks * H + 2047) / 2048;
    seg.prep_group = (int32_t)(want < 1 ? 1 : (want > PREP_GROUP ? PREP_GROUP : want));
    const int64_t grid = (max_chunks + seg.prep_group - 1) / seg.prep_group * H;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(P::NT), P::bytes, stream,
                       static_cast<const TIn *>(q), static_cast<const TIn *>(k), static_cast<const TIn *>(nullptr),
                       g, beta, nullptr, cu, N, T_tot, H, DK, static_cast<TIn *>(nullptr), nullptr, seg);
    return hipGetLastError();
}

template <typename TIn, int C, int NW, int NCT, bool SB = false>
static hipError_t launch_chain_t(const void *v, const float *init, const int32_t *cu, int32_t N, int32_t T_tot,
                                 int32_t H, int32_t dv, void *out, float *fin, SegArgs seg, hipStream_t stream)
{
    typedef ChainCfg<TIn, C, NW, NCT, SB> Q;
    const bool summary = seg.mode == SEG_SUMMARY;
    const int kind = summary ? 1 : (seg.snap ? 2 : 0);
    auto kern = kind == 1 ? kda_chain_kernel<TIn, C, NW, NCT, true, SB>
                          : (kind == 2 ? kda_chain_kernel<TIn, C, NW, NCT, false, SB, true>
                                       : kda_chain_kernel<TIn, C, NW, NCT, false, SB>);
    static std::atomic<uint64_t> lds_set[3];
    if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(kern), (int)Q::bytes, lds_set[kind])) return e;
    const int64_t units = (int64_t)(seg.plan ? seg.num_segs : N) * H;
    const int nblk = (summary ? dv + DK : dv) / Q::BV;
    const int64_t grid = (units + 7) / 8 * 8 * nblk;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Q::NT), Q::bytes, stream, static_cast<const TIn *>(v), init,
                       cu, N, T_tot, H, dv, static_cast<TIn *>(out), fin, seg);
    return hipGetLastError();
}

// ---------------------------------------------------------- segment planning
// One workgroup: segments per sequence (at least one, so that empty sequences
// still produce their final state), exclusive scan, plan entries; and, if
// chunk_off is given, the first chunk of each sequence in chunks of `chunk`
// tokens (chunk_off[N] = total chunks, at most max_chunks); and, if sched is
// given, a dispatch order of the max_segs plan entries (a permutation).
struct PlanArgs {
    int32_t seg_len, max_segs;
    int32_t *plan, *seq_seg, *chunk_off, *sched;   // chunk_off, sched may be nullptr
    int32_t last_len, skip_last;
    int32_t *seq_order;                            // may be nullptr
};
// One plan per workgroup: workgroup b builds plan b (a second plan of the
// same sequences at another granularity costs no extra launch).
__global__ __launch_bounds__(256) void kda_cp_plan_kernel(const int32_t *__restrict__ cu, int32_t N,
                                                          int32_t T_tot, int32_t chunk, int32_t max_chunks,
                                                          PlanArgs a0, PlanArgs a1)
{
    const PlanArgs &pa = blockIdx.x == 0 ? a0 : a1;
    const int32_t seg_len = pa.seg_len, max_segs = pa.max_segs, last_len = pa.last_len, skip_last = pa.skip_last;
    int32_t *const plan = pa.plan, *const seq_seg = pa.seq_seg, *const chunk_off = pa.chunk_off;
    int32_t *const sched = pa.sched, *const seq_order = pa.seq_order;
    __shared__ int64_t scan[256], cscan[256];
    __shared__ int32_t hist[256];
    int64_t carry = 0, ccarry = 0;                     // 64-bit: cu is not trusted
    for (int base = 0; base < N; base += 256) {
        const int n = base + (int)threadIdx.x;
        int32_t t0 = 0, t1 = 0, ns = 0, nc = 0;
        if (n < N) {
            t0 = min(max(cu[n], 0), T_tot);
            t1 = min(max(cu[n + 1], t0), T_tot);
            ns = max(1, (int32_t)(((int64_t)t1 - t0 + seg_len - 1) / seg_len));
            nc = (int32_t)(((int64_t)t1 - t0 + chunk - 1) / chunk);
        }
        scan[threadIdx.x] = ns;
        cscan[threadIdx.x] = nc;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {       // inclusive scans
            const int64_t x = threadIdx.x >= (unsigned)off ? scan[threadIdx.x - off] : 0;
            const int64_t y = threadIdx.x >= (unsigned)off ? cscan[threadIdx.x - off] : 0;
            __syncthreads();
            scan[threadIdx.x] += x;
            cscan[threadIdx.x] += y;
            __syncthreads();
        }
        if (chunk_off && n < N) chunk_off[n] = (int32_t)min(ccarry + cscan[threadIdx.x] - nc, (int64_t)max_chunks);
        const int64_t start = carry + scan[threadIdx.x] - ns;
        if (n < N) {
            // With non-decreasing cu the host bound on max_segs always holds;
            // otherwise segments past it are dropped (memory-safe, result unspecified).
            seq_seg[n] = (int32_t)min(start, (int64_t)max_segs);
            // SEG_LAST: the segment lies in the sequence's last stretch of
            // last_len tokens (a multiple of seg_len), which no later segment follows
            const int64_t nl = last_len > 0 ? max((int64_t)1, ((int64_t)t1 - t0 + last_len - 1) / last_len) : 1;
            for (int s = 0; s < ns && start + s < max_segs; ++s) {
                const int gs = (int)(start + s);
                plan[4 * gs] = n;
                plan[4 * gs + 1] = t0 + s * seg_len;
                plan[4 * gs + 2] = min(t0 + (s + 1) * seg_len, t1);
                plan[4 * gs + 3] = (s == 0 ? SEG_FIRST : 0) |
                                   (last_len > 0 && (int64_t)s * seg_len >= (nl - 1) * last_len ? SEG_LAST : 0);
            }
        }
        carry += scan[255];
        ccarry += cscan[255];
        __syncthreads();
    }
    const int32_t used = (int32_t)min(carry, (int64_t)max_segs);
    if (threadIdx.x == 0) seq_seg[N] = used;
    if (seq_order) {
        // sequences by segment count, most first (counting sort on 256
        // buckets; 255 segments and more share the first): the combine walks
        // the longest chains first
        __syncthreads();   // every seq_seg entry written
        hist[threadIdx.x] = 0;
        __syncthreads();
        auto seq_bucket = [&](int n) { return 255 - min(max(seq_seg[n + 1] - seq_seg[n], 0), 255); };
        for (int n = (int)threadIdx.x; n < N; n += 256) atomicAdd(&hist[seq_bucket(n)], 1);
        __syncthreads();
        const int32_t c = hist[threadIdx.x];
        scan[threadIdx.x] = c;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int64_t x = threadIdx.x >= (unsigned)off ? scan[threadIdx.x - off] : 0;
            __syncthreads();
            scan[threadIdx.x] += x;
            __syncthreads();
        }
        hist[threadIdx.x] = (int32_t)(scan[threadIdx.x] - c);
        __syncthreads();
        for (int n = (int)threadIdx.x; n < N; n += 256) seq_order[atomicAdd(&hist[seq_bucket(n)], 1)] = n;
        __syncthreads();   // hist and scan are reused below
    }
    if (chunk_off && threadIdx.x == 0) chunk_off[N] = (int32_t)min(ccarry, (int64_t)max_chunks);
    for (int gs = used + (int)threadIdx.x; gs < max_segs; gs += 256) {
        plan[4 * gs] = -1;
        plan[4 * gs + 1] = 0;
        plan[4 * gs + 2] = 0;
        plan[4 * gs + 3] = 0;
        if (sched) sched[gs] = gs;
    }
    if (!sched) return;
    // Dispatch order, longest segment first: workgroups start in index order,
    // so the short tail segments fill the gaps the full-length ones leave at
    // the end of a pass.  Counting sort on 256 length buckets (bucket 0 = full
    // length, 255 = empty); the order inside a bucket does not matter, since
    // the segments of one pass are independent.  skip_last: SEG_LAST segments
    // count as empty (a summary pass skips them).
    auto seg_bucket = [&](int gs) {
        int64_t len = (int64_t)plan[4 * gs + 2] - plan[4 * gs + 1];
        if (skip_last && (plan[4 * gs + 3] & SEG_LAST)) len = 0;
        return (int)((seg_len - min(max(len, (int64_t)0), (int64_t)seg_len)) * 255 / seg_len);
    };
    hist[threadIdx.x] = 0;
    __syncthreads();   // also makes this workgroup's plan entries visible below
    for (int gs = (int)threadIdx.x; gs < used; gs += 256) atomicAdd(&hist[seg_bucket(gs)], 1);
    __syncthreads();
    const int32_t cnt = hist[threadIdx.x];
    scan[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int64_t x = threadIdx.x >= (unsigned)off ? scan[threadIdx.x - off] : 0;
        __syncthreads();
        scan[threadIdx.x] += x;
        __syncthreads();
    }
    hist[threadIdx.x] = (int32_t)(scan[threadIdx.x] - cnt);   // bucket start
    __syncthreads();
    for (int gs = (int)threadIdx.x; gs < used; gs += 256) sched[atomicAdd(&hist[seg_bucket(gs)], 1)] = gs;
}

// ------------------------------------------------------ segment combination
// Per (sequence, head, 16 value columns): walk the segments in order,
// S_in(first) = initial state, S_in(s+1) = M_s S_in(s) + S_s^0 on fp32 MFMA,
// writing each segment's entering state.  One workgroup of eight waves per
// (sequence, head, 16 columns), so that a long sequence's chain of steps is
// spread over many compute units: wave w computes row tile w of the next state
// from its own rows of M and the whole current state slice, which every wave
// holds in MFMA accumulator layout and which is exchanged through LDS after
// each step.  A step's operands are loaded two steps ahead, into a ring of
// three register sets.
//   m_src (may be nullptr): M comes from the forward summaries
//     [.][H][DK][dv + DK] (at column dv) instead of seg_out, which then holds
//     S^0 alone in rows of dv floats; MT: M is used transposed.
//   seq_order (may be nullptr): workgroups take the sequences in this order
//     (longest chains first).
//   plan (forward walks only, may be nullptr): the walk stops at the
//     sequence's first SEG_LAST segment, whose entering state is the last one
//     written (the segments after it have no summaries).
//   reverse: the walk goes from the last segment to the first (gradients of
//     the state, which enter a segment at its end): G(last) = init,
//     G(s-1) = R_s G(s) + G_s^0, with R_s = M_s^T when MT.
constexpr int CMB_COLS = 16;
constexpr int CMB_THREADS = 64 * (DK / 16);
struct CmbOps {
    f32x4 m[DK / 16];   // M rows 16 w + lm, columns 16 kb + 4 lj .. + 3 (the k order of Mma<float>)
    f32x4 s0;           // S^0 rows 16 w + 4 lj + i, this lane's column
};
template <bool MT>
__global__ __launch_bounds__(CMB_THREADS) void kda_cp_combine_kernel(const float *__restrict__ init, int32_t N,
                                                                     int32_t H, int32_t dv,
                                                                     const int32_t *__restrict__ seq_seg,
                                                                     const float *seg_out,
                                                                     float *__restrict__ seg_init, int32_t reverse,
                                                                     const int32_t *__restrict__ plan,
                                                                     const int32_t *__restrict__ seq_order,
                                                                     const float *m_src)
{
    typedef Mma<float> M;
    __shared__ __align__(16) f32x4 sS[DK / 16][64];         // the state slice, accumulator layout per row tile
    // the column blocks of one (sequence, head) run on one XCD (workgroups are
    // dealt to the XCDs in turn), so that they read M through one L2
    const int nblk = dv / CMB_COLS;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int64_t unit = (int64_t)(slot / nblk) * 8 + xcd;
    if (unit >= (int64_t)N * H) return;
    const int n = seq_order ? min(max(seq_order[unit / H], 0), N - 1) : (int)(unit / H), h = (int)(unit % H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane >> 4, lm = lane & 15;
    const int col = (slot % nblk) * CMB_COLS + lm;
    // S^0 (and M, unless m_src) in seg_out rows of ld floats; M in rows of ldm
    const int ld = m_src ? dv : dv + DK, ldm = dv + DK;
    // the state slice: every wave holds all of it (rows 16 r + 4 lj + i, column
    // col) and its own row tile in own; both always come from LDS
    f32x4 own, S[DK / 16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        own[i] = init ? init[((int64_t)n * H + h) * DK * dv + (int64_t)(16 * wave + 4 * lj + i) * dv + col] : 0.f;
    sS[wave][lane] = own;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < DK / 16; ++r) S[r] = sS[r][lane];
    own = sS[wave][lane];
    const int s0 = seq_seg[n], s1 = seq_seg[n + 1];
    int ns = s1 - s0;
    if (plan && !reverse)
        for (int it = 0; it < ns - 1; ++it)
            if (plan[4 * (s0 + it) + 3] & SEG_LAST) {
                ns = it + 1;
                break;
            }
    auto seg_of = [&](int it) { return reverse ? s1 - 1 - it : s0 + it; };
    auto fetch = [&](int it, CmbOps &o) {                  // step it's operands (clamped to the last step)
        const int64_t gs = seg_of(min(it, ns - 2));
        const float *src = seg_out + (gs * H + h) * DK * ld;
        const float *msrc = m_src ? m_src + (gs * H + h) * DK * ldm : src;
        if constexpr (MT) {                                // A[i][k] = M[k][i]
#pragma unroll
            for (int kb = 0; kb < DK / 16; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o.m[kb][e] = msrc[(int64_t)(16 * kb + 4 * lj + e) * ldm + dv + 16 * wave + lm];
        } else {
#pragma unroll
            for (int kb = 0; kb < DK / 16; ++kb)
                o.m[kb] = *reinterpret_cast<const f32x4 *>(msrc + (int64_t)(16 * wave + lm) * ldm + dv + 16 * kb + 4 * lj);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) o.s0[i] = src[(int64_t)(16 * wave + 4 * lj + i) * ld + col];
    };
    // step it (it < ns - 1): write S_in of segment it, S <- M S + S^0 from
    // cur, and load step it + 3 into cur's registers afterwards
    auto write_own = [&](int it) {
        float *dst = seg_init + ((int64_t)seg_of(it) * H + h) * DK * dv;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(int64_t)(16 * wave + 4 * lj + i) * dv + col] = own[i];
    };
    auto step = [&](int it, CmbOps &cur) {
        write_own(it);
        f32x4 a = cur.s0, b = zero4();                      // two accumulation chains
#pragma unroll
        for (int kb = 0; kb < DK / 16; kb += 2) {
            a = M::mma(cur.m[kb], S[kb], a);
            b = M::mma(cur.m[kb + 1], S[kb + 1], b);
        }
        fetch(it + 3, cur);
        asm volatile("" ::: "memory");                     // keeps the loads here (not sunk into a later step)
        __syncthreads();                                   // every wave's reads of the previous slice are done
        own = a + b;
        sS[wave][lane] = own;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < DK / 16; ++r) S[r] = sS[r][lane];
    };
    // whole rounds of three steps with no exit inside (the wait for each
    // step's operands then stays exact across the loop's back edge), then the
    // remaining steps and the last segment's entering state
    CmbOps o0, o1, o2;
    const int nst = ns - 1;
    if (nst > 0) {
        fetch(0, o0);
        fetch(1, o1);
        fetch(2, o2);
    }
    int it = 0;
    for (; it + 3 <= nst; it += 3) {
        step(it, o0);
        step(it + 1, o1);
        step(it + 2, o2);
    }
    if (it < nst) step(it, o0);
    if (it + 1 < nst) step(it + 1, o1);
    if (ns > 0) write_own(ns - 1);
}

}  // namespace kda

// Dispatch on (dtype, chunk, dv_block); returns hipErrorInvalidValue for an
// unsupported combination (the host API validates before calling).
extern "C" hipError_t kda_launch_prefill(int bf16, int chunk, int dv_block,
                                         const void *q, const void *k, const void *v,
                                         const float *g, const float *beta, const float *init,
                                         const int32_t *cu, int32_t N, int32_t T_tot, int32_t H,
                                         int32_t dv, void *out, float *fin, float *snap, int32_t snap_every,
                                         int32_t max_snaps, const int32_t *snap_chunk_off, hipStream_t stream)
{
    using namespace kda;
    const SegArgs seg = {nullptr, 0, SEG_OUTPUT, nullptr, nullptr, snap_chunk_off, nullptr, snap, snap_every, max_snaps, nullptr,
                         nullptr, 0, 0, 0};
    if (snap) {   // snapshots: 32-token chunks, 64-column value blocks
        if (chunk != 32 || dv_block != 64) return hipErrorInvalidValue;
        if (bf16) return launch_prefill_t<bf16_t, 32, 4, MODE_SNAP>(q, k, v, g, beta, init, cu, N, T_tot, H, dv, out, fin, seg, stream);
        return launch_prefill_t<float, 32, 4, MODE_SNAP>(q, k, v, g, beta, init, cu, N, T_tot, H, dv, out, fin, seg, stream);
    }
#define KDA_CASE(TT, CC, NWW)                                                                    \
    if (chunk == CC && dv_block == 16 * NWW)                                                       \
        return launch_prefill_t<TT, CC, NWW, MODE_FUSED>(q, k, v, g, beta, init, cu, N, T_tot, H, dv, out, fin, seg, stream);
    if (bf16) {
        KDA_CASE(bf16_t, 32, 1) KDA_CASE(bf16_t, 32, 2) KDA_CASE(bf16_t, 32, 4) KDA_CASE(bf16_t, 32, 8)
        KDA_CASE(bf16_t, 64, 2) KDA_CASE(bf16_t, 64, 4) KDA_CASE(bf16_t, 64, 8)
    } else {
        KDA_CASE(float, 32, 1) KDA_CASE(float, 32, 2) KDA_CASE(float, 32, 4) KDA_CASE(float, 32, 8)
        KDA_CASE(float, 16, 1) KDA_CASE(float, 16, 2) KDA_CASE(float, 16, 4) KDA_CASE(float, 16, 8)
    }
#undef KDA_CASE
    return hipErrorInvalidValue;
}

// last_len: SEG_LAST marks the segments in each sequence's last stretch of
// last_len tokens (a multiple of seg_len; 0 = seg_len: the last segment;
// negative: no segment is marked, so a summary pass covers them all);
// skip_last: those segments go last in the dispatch order; seq_order
// (optional, [N]): the sequences by segment count, most first.  A second plan
// (plan2 != nullptr, with its own seg_len2 ... seq_order2) is built by a
// second workgroup of the same launch.
extern "C" hipError_t kda_launch_cp_plan(const int32_t *cu, int32_t N, int32_t T_tot, int32_t seg_len,
                                         int32_t max_segs, int32_t *plan, int32_t *seq_seg, int32_t chunk,
                                         int32_t max_chunks, int32_t *chunk_off, int32_t *sched,
                                         int32_t last_len, int32_t skip_last, int32_t *seq_order,
                                         int32_t seg_len2, int32_t max_segs2, int32_t *plan2, int32_t *seq_seg2,
                                         int32_t *sched2, int32_t last_len2, int32_t skip_last2,
                                         int32_t *seq_order2, hipStream_t stream)
{
    auto args = [](int32_t sl, int32_t ms, int32_t *p, int32_t *ss, int32_t *co, int32_t *sc, int32_t ll,
                   int32_t sk, int32_t *so, kda::PlanArgs *a) {
        if (ll == 0) ll = sl;
        if (sl <= 0 || (ll > 0 && ll % sl)) return false;
        *a = {sl, ms, p, ss, co, sc, ll, sk, so};
        return true;
    };
    kda::PlanArgs a0, a1;
    if (!args(seg_len, max_segs, plan, seq_seg, chunk_off, sched, last_len, skip_last, seq_order, &a0))
        return hipErrorInvalidValue;
    a1 = a0;
    if (plan2 && !args(seg_len2, max_segs2, plan2, seq_seg2, nullptr, sched2, last_len2, skip_last2, seq_order2, &a1))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kda::kda_cp_plan_kernel, dim3(plan2 ? 2 : 1), dim3(256), 0, stream, cu, N, T_tot, chunk,
                       max_chunks, a0, a1);
    return hipGetLastError();
}

// Chunk-operand pass: images of every (chunk, head), 32-token chunks.
extern "C" hipError_t kda_launch_chunk_prep(int bf16, const void *q, const void *k, const float *g,
                                            const float *beta, const int32_t *cu, int32_t N, int32_t T_tot,
                                            int32_t H, const int32_t *chunk_off, int64_t max_chunks, void *img,
                                            hipStream_t stream)
{
    using namespace kda;
    if (max_chunks < 1 || max_chunks > 0x7fffffff) return hipErrorInvalidValue;
    SegArgs seg = {nullptr, 0, SEG_OUTPUT, nullptr, nullptr, chunk_off, static_cast<f32x4 *>(img), nullptr, 0, 0, nullptr,
                   nullptr, 0, 0, PREP_GROUP, (int32_t)max_chunks};
    if (bf16) return launch_prep_t<bf16_t, 32>(q, k, g, beta, cu, N, T_tot, H, max_chunks, seg, stream);
    return launch_prep_t<float, 32>(q, k, g, beta, cu, N, T_tot, H, max_chunks, seg, stream);
}

// State-chain pass over the images, value blocks of dv_block columns (64,
// 128, or 256 for a summary's value + transition columns in one block);
// plan, mode, seg_init and seg_out as for kda_launch_prefill.
extern "C" hipError_t kda_launch_chain(int bf16, int dv_block, const void *v, const float *init, const int32_t *cu, int32_t N,
                                       int32_t T_tot, int32_t H, int32_t dv, void *out, float *fin,
                                       const int32_t *plan, int32_t num_segs, int32_t mode, const float *seg_init,
                                       float *seg_out, const int32_t *chunk_off, const void *img,
                                       const int32_t *sched, float *snap, const int32_t *init_seq_seg,
                                       int32_t init_unit, int32_t init_units, hipStream_t stream)
{
    using namespace kda;
    if (init_seq_seg && (init_unit <= 0 || init_units <= 0)) return hipErrorInvalidValue;
    SegArgs seg = {plan, num_segs, mode, seg_init, seg_out, chunk_off,
                   const_cast<f32x4 *>(static_cast<const f32x4 *>(img)), mode == SEG_SUMMARY ? nullptr : snap, 0, 0,
                   sched, init_seq_seg, init_unit, init_units, 0};
    // bf16: 256 columns (segment summaries) as 8 waves x 2 tiles, double
    // buffered; 128 columns (outputs) as 4 waves x 2 tiles, single buffered,
    // two workgroups per compute unit (two tiles per wave share every operand
    // fragment; the second workgroup covers the waits of the first); fp32
    // images are twice as large and their buffers fit the LDS at 64 columns only
    // with state stores: 64 columns per workgroup (the two-tile form has no registers left for them)
    if (bf16 && seg.snap) return launch_chain_t<bf16_t, 32, 4, 1>(v, init, cu, N, T_tot, H, dv, out, fin, seg, stream);
    if (bf16 && dv_block == 256) return launch_chain_t<bf16_t, 32, 8, 2>(v, init, cu, N, T_tot, H, dv, out, fin, seg, stream);
    if (bf16 && dv_block == 128) return launch_chain_t<bf16_t, 32, 4, 2, true>(v, init, cu, N, T_tot, H, dv, out, fin, seg, stream);
    if (dv_block != 64 && dv_block != 128 && dv_block != 256) return hipErrorInvalidValue;
    if (bf16) return launch_chain_t<bf16_t, 32, 4, 1>(v, init, cu, N, T_tot, H, dv, out, fin, seg, stream);
    return launch_chain_t<float, 32, 4, 1>(v, init, cu, N, T_tot, H, dv, out, fin, seg, stream);
}

extern "C" size_t kda_chunk_image_bytes(int bf16)
{
    return bf16 ? kda::ChunkImage<kda::bf16_t, 32>::BYTES : kda::ChunkImage<float, 32>::BYTES;
}

extern "C" hipError_t kda_launch_cp_combine(const float *init, int32_t N, int32_t H, int32_t dv,
                                            const int32_t *seq_seg, const float *seg_out, float *seg_init,
                                            int32_t reverse, const int32_t *plan, const int32_t *seq_order,
                                            const float *m_src, int32_t m_trans, hipStream_t stream)
{
    const int64_t grid = ((int64_t)N * H + 7) / 8 * 8 * (dv / kda::CMB_COLS);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (m_trans && !m_src) return hipErrorInvalidValue;
    hipLaunchKernelGGL(m_trans ? kda::kda_cp_combine_kernel<true> : kda::kda_cp_combine_kernel<false>,
                       dim3((unsigned)grid), dim3(kda::CMB_THREADS), 0, stream, init, N, H, dv, seq_seg, seg_out,
                       seg_init, reverse, plan, seq_order, m_src);
    return hipGetLastError();
}
