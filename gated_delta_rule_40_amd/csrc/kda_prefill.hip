// kda_prefill.hip -- chunked KDA prefill for gfx950.
//
// The recurrence (page "Kimi K3 把 3T 级模型、百万上下文和 Agent 训练接成一套系统",
// ailearn.mscapital.top/kimi-k3.html, card "KDA 单头递归"), per (sequence, head):
//     S_t = (I - b_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t.
//
// Chunked form evaluated here (derived from that recurrence; C tokens per
// chunk, entering state S0, Gamma_r = sum_{i<=r} g_i, all per key channel):
//     X   = Diag(b) (V - K+ S0)                           K+ = K (.) e^Gamma
//     (I + Diag(b) A) W = X,  A_ri = sum_c k_rc k_ic e^(Gamma_rc - Gamma_ic), i < r
//     O   = Q+ S0 + P W,      P_ri = sum_c q_rc k_ic e^(Gamma_rc - Gamma_ic), i <= r
//     S_C = Diag(e^Gamma_C) S0 + K^T W                    K^ = K (.) e^(Gamma_C - Gamma)
// A and P ("Gram" tiles) are built per 16-token sub-tile pair with decay
// factors referenced to sub-tile boundaries (card "g ∈ (-5, 0)": inside a
// 16-token tile the cumulative scaling stays within bf16 range), so every
// factor is <= 1 except the diagonal sub-tile's column factor (<= e^80 for
// g >= -5).  W comes from block forward substitution over the sub-tiles with
// the 16x16 diagonal blocks inverted once per chunk.
//
// Precision (bf16 q/k/v): all state-dependent contractions run on fp16 MFMA
// operands with fp32 accumulation; the fp32 state, X and W are converted with
// exact per-column power-of-two scales, so their range is unrestricted.  The
// Gram tiles use fp16 operands when every sub-tile's decay span is <= 8
// (column factors <= e^8) and fp32 MFMA otherwise (chosen per chunk).  fp32
// q/k/v use fp32 MFMA throughout.
//
// Work decomposition: one workgroup per (sequence, head, block of BV value
// columns), NW = BV/16 waves.  Each wave owns 16 columns of the fp32 state,
// kept in MFMA accumulator registers for the whole sequence.  Per chunk:
//   1. decay prep (all threads): sub-tile gate sums, per-token cumulative
//      products, decayed operands written to LDS;
//   2. Gram tiles A, P on MFMA (jobs spread over the waves);
//   3. 16x16 diagonal inverses (VALU forward substitution), value tile load;
//   4. state-dependent chain per wave: X, W, O and the state update on MFMA;
//   5. coalesced store of the output tile.
// Ragged chunks are zero-padded (k = q = v = 0, g = 0, b = 0), which leaves
// the result exact.
#include <type_traits>

#include "kda_device.hpp"

namespace kda {

constexpr int DK = 128;
constexpr int SUB = 16;
constexpr float SPAN_FAST = 8.f;   // max sub-tile decay span for fp16 Gram operands
// fp16 Gram operands: row operands are stored x2^5 and column factors x2^-5
// (exact, cancelling) so that row values keep clear of fp16 subnormals while
// column values (up to |k| e^8) stay below the fp16 maximum.
constexpr float GRAM16_ROW = 32.f;

template <typename TIn, int C, int NW>
struct PrefillCfg {
    static constexpr bool kIn16 = !std::is_same<TIn, float>::value;
    typedef typename std::conditional<kIn16, f16_t, float>::type OpT;   // chain operands
    static constexpr int BV = 16 * NW;
    static constexpr int NT = 64 * NW;
    static constexpr int NSUB = C / SUB;
    static constexpr int NPAIR = NSUB * (NSUB + 1) / 2;
    static constexpr int KB = Mma<OpT>::KB;
    static_assert(C % KB == 0, "chunk must be a multiple of the MFMA K-block");
    static_assert(NSUB >= 1 && NSUB <= 4, "chunk of 16..64 tokens");

    // row strides (elements), each row padded by 16 bytes against bank conflicts
    static constexpr int LDK = DK + 16 / (int)sizeof(OpT);     // [C][DK] OpT tiles
    static constexpr int LDC = C + 16 / (int)sizeof(OpT);      // [*][C] OpT tiles
    static constexpr int LDK32 = DK + 4;                       // [C][DK] fp32 tiles
    static constexpr int LDV = BV + 16 / (int)sizeof(TIn);     // value / output tiles
    static constexpr int LDI = SUB + 16 / (int)sizeof(OpT);    // diagonal inverses

    static constexpr size_t tileK = sizeof(OpT) * C * LDK;
    static constexpr size_t tileK32 = sizeof(float) * C * LDK32;
    // Region G/B: Gram inputs [Kr][Qr][KD] (OpT) then chain operands
    // [-K+][Q+][K^T] (OpT).  For bf16 input the fp32 Gram inputs of a
    // strong-decay chunk [Kr32][Qr32][KD32] overlay the whole region.
    static constexpr size_t offKr = 0;
    static constexpr size_t offQr = offKr + tileK;
    static constexpr size_t offKD = offQr + tileK;
    static constexpr size_t offNKp = offKD + tileK;
    static constexpr size_t offQp = offNKp + tileK;
    static constexpr size_t offKhT = offQp + tileK;
    static constexpr size_t endGB = offKhT + sizeof(OpT) * DK * LDC;
    static constexpr size_t offKr32 = 0;
    static constexpr size_t offQr32 = offKr32 + tileK32;
    static constexpr size_t offKD32 = offQr32 + tileK32;
    static_assert(!kIn16 || offKD32 + tileK32 <= endGB, "fp32 Gram inputs must fit the region");
    // Region D (after the Gram step): value tile, output tile, inverses; inside [Kr][Qr][KD]
    static constexpr size_t offV = 0;
    static constexpr size_t offO = offV + sizeof(TIn) * C * LDV;
    static constexpr size_t offInv = offO + sizeof(TIn) * C * LDV;
    static_assert(offInv + sizeof(OpT) * NSUB * SUB * LDI <= offNKp, "region D must fit");
    // Region C: Gram outputs
    static constexpr size_t offAd = endGB;                                   // fp32 [NSUB*16][17]
    static constexpr size_t offNs = offAd + sizeof(float) * NSUB * SUB * 17;  // OpT [C][LDC]
    static constexpr size_t offP = offNs + sizeof(OpT) * C * LDC;            // OpT [C][LDC]
    static constexpr size_t endC = offP + sizeof(OpT) * C * LDC;
    // small fp32 tables
    static constexpr size_t offF = (endC + 15) / 16 * 16;                    // [NSUB][DK]
    static constexpr size_t offH = offF + sizeof(float) * NSUB * DK;         // [NPAIR][DK]
    static constexpr size_t offGam = offH + sizeof(float) * NPAIR * DK;      // [DK]
    static constexpr size_t offBeta = offGam + sizeof(float) * DK;           // [C]
    static constexpr size_t offInvS = offBeta + sizeof(float) * C;           // [NSUB]
    static constexpr size_t bytes = offInvS + sizeof(float) * NSUB;
    static_assert(bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

// sub-tile pair p -> (a, b), b <= a
__device__ __forceinline__ void pair_of(int p, int &a, int &b) {
    a = 0;
    while ((a + 1) * (a + 2) / 2 <= p) ++a;
    b = p - a * (a + 1) / 2;
}

// Gram tiles A (strictly lower) and P (lower incl.) for every sub-tile pair,
// operands of type GT in LDS with row stride ld; the column operand of pair
// (a, b) is KD of sub-tile b scaled per channel by H(a, b).
template <typename GT, typename OpT, int C, int NW>
__device__ __forceinline__ void gram_tiles(const GT *sKr, const GT *sQr, const GT *sKD, int ld,
                                           const float *sH, const float *sBeta, float *sAd,
                                           OpT *sNs, OpT *sP, int ldc, int wave, int lj, int lm)
{
    typedef Mma<GT> G;
    constexpr int NSUB = C / SUB, NPAIR = NSUB * (NSUB + 1) / 2;
    constexpr int KBc = Mma<OpT>::KB;    // K-block of the P W contraction in the chain
    for (int p = wave; p < NPAIR; p += NW) {
        int a, b;
        pair_of(p, a, b);
        f32x4 accA = zero4(), accP = zero4();
        const GT *rowKr = sKr + (a * SUB + lm) * ld;
        const GT *rowQr = sQr + (a * SUB + lm) * ld;
        const GT *rowKD = sKD + (b * SUB + lm) * ld;
        const float *hs = sH + p * DK;
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += G::KB) {
            const typename G::frag bf = G::load_scaled(rowKD, hs, k0, lj);
            accA = G::mma(G::load(rowKr, k0, lj), bf, accA);
            accP = G::mma(G::load(rowQr, k0, lj), bf, accP);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = 4 * lj + i;                 // row within sub-tile a
            const int r = a * SUB + rl, cc = b * SUB + lm;
            float av = accA[i], pv = accP[i];
            if (a == b) {
                if (lm >= rl) av = 0.f;
                if (lm > rl) pv = 0.f;
            }
            const float nv = sBeta[r] * av;            // N = Diag(beta) A
            if (a == b)
                sAd[(a * SUB + rl) * 17 + lm] = nv;
            else
                sNs[r * ldc + cc] = from_f<OpT>(-nv);
            sP[r * ldc + cc] = from_f<OpT>(pv);
            if (KBc == 32 && a == b && (a & 1) == 0 && a + 1 < NSUB)
                sP[r * ldc + cc + SUB] = from_f<OpT>(0.f);  // a K-block pairs sub-tiles a, a+1
        }
    }
}

template <typename TIn, int C, int NW>
__global__ __launch_bounds__(64 * NW) void kda_prefill_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *initial_state, const int32_t *__restrict__ cu_seqlens,
    int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dv,
    TIn *__restrict__ out, float *final_state)
{
    typedef PrefillCfg<TIn, C, NW> P;
    typedef typename P::OpT OpT;
    typedef Mma<OpT> M;
    constexpr bool kIn16 = P::kIn16;
    constexpr int NSUB = P::NSUB, BV = P::BV, NT = P::NT, KB = P::KB;
    constexpr int LDK = P::LDK, LDC = P::LDC, LDK32 = P::LDK32, LDV = P::LDV, LDI = P::LDI;

    extern __shared__ __align__(16) unsigned char smem[];
    OpT *sKr = reinterpret_cast<OpT *>(smem + P::offKr);
    OpT *sQr = reinterpret_cast<OpT *>(smem + P::offQr);
    OpT *sKD = reinterpret_cast<OpT *>(smem + P::offKD);
    float *sKr32 = reinterpret_cast<float *>(smem + P::offKr32);
    float *sQr32 = reinterpret_cast<float *>(smem + P::offQr32);
    float *sKD32 = reinterpret_cast<float *>(smem + P::offKD32);
    OpT *sNKp = reinterpret_cast<OpT *>(smem + P::offNKp);
    OpT *sQp = reinterpret_cast<OpT *>(smem + P::offQp);
    OpT *sKhT = reinterpret_cast<OpT *>(smem + P::offKhT);
    TIn *sV = reinterpret_cast<TIn *>(smem + P::offV);
    TIn *sO = reinterpret_cast<TIn *>(smem + P::offO);
    OpT *sInv = reinterpret_cast<OpT *>(smem + P::offInv);
    float *sAd = reinterpret_cast<float *>(smem + P::offAd);
    OpT *sNs = reinterpret_cast<OpT *>(smem + P::offNs);
    OpT *sP = reinterpret_cast<OpT *>(smem + P::offP);
    float *sF = reinterpret_cast<float *>(smem + P::offF);
    float *sH = reinterpret_cast<float *>(smem + P::offH);
    float *sGam = reinterpret_cast<float *>(smem + P::offGam);
    float *sBeta = reinterpret_cast<float *>(smem + P::offBeta);
    float *sInvS = reinterpret_cast<float *>(smem + P::offInvS);

    // ---- workgroup -> (sequence, head, value block); blocks of one unit share an XCD
    const int nblk = dv / BV;
    const int wg = blockIdx.x;
    const int xcd = wg & 7, slot = wg >> 3;
    const int vb = slot % nblk;
    const int64_t unit = (int64_t)(slot / nblk) * 8 + xcd;
    if (unit >= (int64_t)num_seqs * num_heads) return;
    const int n = (int)(unit / num_heads), h = (int)(unit % num_heads);
    const int dv0 = vb * BV;

    int t_start = cu_seqlens[n], t_end = cu_seqlens[n + 1];
    t_start = min(max(t_start, 0), total_tokens);
    t_end = min(max(t_end, t_start), total_tokens);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lj = lane >> 4, lm = lane & 15;
    const int H = num_heads;
    const int64_t rowK = (int64_t)H * DK;      // token stride of q, k, g
    const int64_t rowV = (int64_t)H * dv;      // token stride of v, out
    const int64_t hK = (int64_t)h * DK;

    // ---- state slice of this wave: rows 16r + 4*lj + i, column dv0 + 16*wave + lm
    f32x4 S[DK / 16];
    const int col = dv0 + 16 * wave + lm;
    const int64_t sbase = unit * (int64_t)DK * dv;
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[r][i] = initial_state ? initial_state[sbase + (int64_t)(16 * r + 4 * lj + i) * dv + col] : 0.f;

    for (int c0 = t_start; c0 < t_end; c0 += C) {
        const int L = min(C, t_end - c0);        // valid tokens in this chunk
        __syncthreads();                          // previous chunk done with all LDS

        // ---- 1a. sub-tile gate sums -> F_a = exp(sum); beta; strong-decay test
        int strong = 0;
        for (int item = tid; item < NSUB * (DK / 2); item += NT) {
            const int a = item / (DK / 2), c = 2 * (item % (DK / 2));
            float s0 = 0.f, s1 = 0.f;
            for (int rr = 0; rr < SUB; ++rr) {
                const int r = a * SUB + rr;
                if (r < L) {
                    const f32x2 gg = *reinterpret_cast<const f32x2 *>(g + (int64_t)(c0 + r) * rowK + hK + c);
                    s0 += gg[0];
                    s1 += gg[1];
                }
            }
            strong |= (s0 < -SPAN_FAST) | (s1 < -SPAN_FAST);
            sF[a * DK + c] = __expf(s0);
            sF[a * DK + c + 1] = __expf(s1);
        }
        for (int r = tid; r < C; r += NT)
            sBeta[r] = (r < L) ? beta[(int64_t)(c0 + r) * H + h] : 0.f;
        // fp16 Gram operands need every column factor <= e^8; fp32 input always uses fp32
        const bool gram32 = !kIn16 || __syncthreads_or(strong);
        if (!kIn16) __syncthreads();

        // ---- 1b. tables: H(a,b) = prod_{b<s<a} F_s (b < a), 1/F_a (b = a); gamma = prod F
        for (int e = tid; e < (P::NPAIR + 1) * DK; e += NT) {
            const int p = e / DK, c = e % DK;
            if (p == P::NPAIR) {
                float gm = 1.f;
                for (int s = 0; s < NSUB; ++s) gm *= sF[s * DK + c];
                sGam[c] = gm;
            } else {
                int a, b;
                pair_of(p, a, b);
                float hv;
                if (b == a) {
                    hv = 1.f / sF[a * DK + c];
                } else {
                    hv = 1.f;
                    for (int s = b + 1; s < a; ++s) hv *= sF[s * DK + c];
                }
                sH[p * DK + c] = gram32 ? hv : hv * (1.f / GRAM16_ROW);
            }
        }

        // ---- 1c. per-token decayed operands (Gram inputs; chain operands unless
        //          the Gram inputs are fp32 and overlay them)
        auto decay_prep = [&](bool gram_inputs, bool chain_ops, bool as32) {
            for (int item = tid; item < NSUB * (DK / 2); item += NT) {
                const int a = item / (DK / 2), c = 2 * (item % (DK / 2));
                f32x2 erho = {1.f, 1.f}, suff = {1.f, 1.f};
                for (int s = 0; s < a; ++s) { erho[0] *= sF[s * DK + c]; erho[1] *= sF[s * DK + c + 1]; }
                for (int s = a + 1; s < NSUB; ++s) { suff[0] *= sF[s * DK + c]; suff[1] *= sF[s * DK + c + 1]; }
                f32x2 al[SUB], kk[SUB];
#pragma unroll
                for (int rr = 0; rr < SUB; ++rr) {
                    const int r = a * SUB + rr;
                    if (r < L) {
                        const int64_t off = (int64_t)(c0 + r) * rowK + hK + c;
                        const f32x2 gg = *reinterpret_cast<const f32x2 *>(g + off);
                        al[rr][0] = __expf(gg[0]);
                        al[rr][1] = __expf(gg[1]);
                        kk[rr] = load_pair(k + off);
                    } else {
                        al[rr] = f32x2{1.f, 1.f};
                        kk[rr] = f32x2{0.f, 0.f};
                    }
                }
                // backward products: D_r = prod_{s > r in sub-tile} alpha_s
                f32x2 D = {1.f, 1.f};
#pragma unroll
                for (int rr = SUB - 1; rr >= 0; --rr) {
                    const int r = a * SUB + rr;
                    const float kd0 = kk[rr][0] * D[0], kd1 = kk[rr][1] * D[1];
                    if (gram_inputs) {
                        if (as32) store_pair(sKD32 + r * LDK32 + c, kd0, kd1);
                        else store_pair(sKD + r * LDK + c, kd0, kd1);
                    }
                    if (chain_ops) {
                        sKhT[c * LDC + r] = from_f<OpT>(kd0 * suff[0]);
                        sKhT[(c + 1) * LDC + r] = from_f<OpT>(kd1 * suff[1]);
                    }
                    D = D * al[rr];
                }
                // forward products: R_r = prod_{s <= r in sub-tile} alpha_s
                f32x2 R = {1.f, 1.f};
#pragma unroll
                for (int rr = 0; rr < SUB; ++rr) {
                    const int r = a * SUB + rr;
                    f32x2 qq = {0.f, 0.f};
                    if (r < L) qq = load_pair(q + (int64_t)(c0 + r) * rowK + hK + c);
                    R = R * al[rr];
                    const float kr0 = kk[rr][0] * R[0], kr1 = kk[rr][1] * R[1];
                    const float qr0 = qq[0] * R[0], qr1 = qq[1] * R[1];
                    if (gram_inputs) {
                        if (as32) {
                            store_pair(sKr32 + r * LDK32 + c, kr0, kr1);
                            store_pair(sQr32 + r * LDK32 + c, qr0, qr1);
                        } else {
                            store_pair(sKr + r * LDK + c, kr0 * GRAM16_ROW, kr1 * GRAM16_ROW);
                            store_pair(sQr + r * LDK + c, qr0 * GRAM16_ROW, qr1 * GRAM16_ROW);
                        }
                    }
                    if (chain_ops) {
                        store_pair(sNKp + r * LDK + c, -kr0 * erho[0], -kr1 * erho[1]);
                        store_pair(sQp + r * LDK + c, qr0 * erho[0], qr1 * erho[1]);
                    }
                }
            }
        };
        const bool overlay = kIn16 && gram32;     // fp32 Gram inputs overlay the chain operands
        decay_prep(true, !overlay, gram32);
        __syncthreads();

        // ---- 2. Gram tiles
        if (gram32)
            gram_tiles<float, OpT, C, NW>(sKr32, sQr32, sKD32, LDK32, sH, sBeta, sAd, sNs, sP, LDC, wave, lj, lm);
        else
            gram_tiles<OpT, OpT, C, NW>(sKr, sQr, sKD, LDK, sH, sBeta, sAd, sNs, sP, LDC, wave, lj, lm);
        __syncthreads();

        // ---- 3. chain operands after an fp32 Gram; diagonal inverses; value tile
        if (overlay) decay_prep(false, true, false);
        for (int e = tid; e < NSUB * SUB; e += NT) {
            const int a = e / SUB, nc = e % SUB;
            const float *Nb = sAd + a * SUB * 17;
            float x[SUB];
#pragma unroll
            for (int r = 0; r < SUB; ++r) x[r] = (r == nc) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < SUB; ++s)
#pragma unroll
                for (int r = s + 1; r < SUB; ++r) x[r] -= Nb[r * 17 + s] * x[s];
            // keep fp16 operands in range: scale the block down if it exceeds 2^14
            float sc = 1.f;
            if (kIn16) {
                float m = 0.f;
#pragma unroll
                for (int r = 0; r < SUB; ++r) m = fmaxf(m, fabsf(x[r]));
                m = fmaxf(m, __shfl_xor(m, 1));
                m = fmaxf(m, __shfl_xor(m, 2));
                m = fmaxf(m, __shfl_xor(m, 4));
                m = fmaxf(m, __shfl_xor(m, 8));
                if (m > 16384.f) sc = pow2_scale(m);
                if (nc == 0) sInvS[a] = pow2_inv(sc);
            } else if (nc == 0) {
                sInvS[a] = 1.f;
            }
#pragma unroll
            for (int r = 0; r < SUB; ++r) sInv[(a * SUB + r) * LDI + nc] = from_f<OpT>(x[r] * sc);
        }
        {
            constexpr int VEC = 16 / sizeof(TIn);          // elements per 16-byte vector
            constexpr int VPR = BV / VEC;                  // vectors per token row
            for (int e = tid; e < C * VPR; e += NT) {
                const int r = e / VPR, cv = (e % VPR) * VEC;
                f32x4 val = zero4();
                if (r < L)
                    val = *reinterpret_cast<const f32x4 *>(v + (int64_t)(c0 + r) * rowV + (int64_t)h * dv + dv0 + cv);
                *reinterpret_cast<f32x4 *>(sV + r * LDV + cv) = val;
            }
        }
        __syncthreads();

        // ---- 4. state-dependent chain (this wave's 16 columns)
        {
            const int vc = 16 * wave + lm;                 // column within the value block
            // state operand, scaled per column into fp16 range
            float sS = 1.f, isS = 1.f;
            if (kIn16) {
                float m = 0.f;
#pragma unroll
                for (int r = 0; r < DK / 16; ++r) m = fmaxf(m, absmax4(S[r]));
                sS = pow2_scale(colmax(m));
                isS = pow2_inv(sS);
            }
            typename M::frag Sf[DK / KB];
#pragma unroll
            for (int kb = 0; kb < DK / KB; ++kb) Sf[kb] = M::from_acc(&S[kb * (KB / 16)], sS);

            // X = Diag(beta) (V - K+ S0)
            f32x4 X[NSUB];
#pragma unroll
            for (int mt = 0; mt < NSUB; ++mt) {
                f32x4 t = zero4();
                const OpT *rowA = sNKp + (mt * SUB + lm) * LDK;
#pragma unroll
                for (int kb = 0; kb < DK / KB; ++kb) t = M::mma(M::load(rowA, kb * KB, lj), Sf[kb], t);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = mt * SUB + 4 * lj + i;
                    X[mt][i] = sBeta[r] * (to_f(sV[r * LDV + vc]) + t[i] * isS);
                }
            }
            // W by forward substitution over sub-tiles (fp16 operands, per-tile column scales)
            f32x4 W[NSUB];
            typename M::frag16 W16[NSUB];
            float iW[NSUB];
            float wmax = 0.f;
#pragma unroll
            for (int a = 0; a < NSUB; ++a) {
                f32x4 acc = X[a];
                const OpT *rowN = sNs + (a * SUB + lm) * LDC;
#pragma unroll
                for (int b = 0; b < a; ++b) {
                    const f32x4 t = M::mma16(M::load16(rowN, b * SUB, lj), W16[b], zero4());
                    acc += t * iW[b];
                }
                float sR = 1.f, isR = 1.f;
                if (kIn16) { sR = pow2_scale(colmax(absmax4(acc))); isR = pow2_inv(sR); }
                const f32x4 t = M::mma16(M::load16(sInv + (a * SUB + lm) * LDI, 0, lj), M::from_acc16(acc, sR), zero4());
                W[a] = t * (isR * sInvS[a]);
                float sW = 1.f;
                if (kIn16) {
                    const float m = colmax(absmax4(W[a]));
                    wmax = fmaxf(wmax, m);
                    sW = pow2_scale(m);
                }
                iW[a] = pow2_inv(sW);
                W16[a] = M::from_acc16(W[a], sW);
            }
            float sWc = 1.f, isWc = 1.f;
            if (kIn16) { sWc = pow2_scale(wmax); isWc = pow2_inv(sWc); }
            typename M::frag Wf[C / KB];
#pragma unroll
            for (int kb = 0; kb < C / KB; ++kb) Wf[kb] = M::from_acc(&W[kb * (KB / 16)], sWc);

            // O = Q+ S0 + P W
#pragma unroll
            for (int mt = 0; mt < NSUB; ++mt) {
                f32x4 o1 = zero4(), o2 = zero4();
                const OpT *rowQ = sQp + (mt * SUB + lm) * LDK;
#pragma unroll
                for (int kb = 0; kb < DK / KB; ++kb) o1 = M::mma(M::load(rowQ, kb * KB, lj), Sf[kb], o1);
                const OpT *rowP = sP + (mt * SUB + lm) * LDC;
#pragma unroll
                for (int kb = 0; kb < C / KB; ++kb)
                    if (kb * KB <= mt * SUB + SUB - 1) o2 = M::mma(M::load(rowP, kb * KB, lj), Wf[kb], o2);
                const f32x4 o = o1 * isS + o2 * isWc;
#pragma unroll
                for (int i = 0; i < 4; ++i) sO[(mt * SUB + 4 * lj + i) * LDV + vc] = from_f<TIn>(o[i]);
            }
            // S = Diag(gamma) S0 + K^T W
#pragma unroll
            for (int r = 0; r < DK / 16; ++r) {
                f32x4 t = zero4();
                const OpT *rowK = sKhT + (16 * r + lm) * LDC;
#pragma unroll
                for (int kb = 0; kb < C / KB; ++kb) t = M::mma(M::load(rowK, kb * KB, lj), Wf[kb], t);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[r][i] = S[r][i] * sGam[16 * r + 4 * lj + i] + t[i] * isWc;
            }
        }
        __syncthreads();

        // ---- 5. output tile -> global (valid tokens only)
        {
            constexpr int VEC = 16 / sizeof(TIn);
            constexpr int VPR = BV / VEC;
            for (int e = tid; e < C * VPR; e += NT) {
                const int r = e / VPR, cv = (e % VPR) * VEC;
                if (r < L)
                    *reinterpret_cast<f32x4 *>(out + (int64_t)(c0 + r) * rowV + (int64_t)h * dv + dv0 + cv) =
                        *reinterpret_cast<const f32x4 *>(sO + r * LDV + cv);
            }
        }
    }

    if (final_state) {
#pragma unroll
        for (int r = 0; r < DK / 16; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                final_state[sbase + (int64_t)(16 * r + 4 * lj + i) * dv + col] = S[r][i];
    }
}

// ------------------------------------------------------------------ launch
template <typename TIn, int C, int NW>
static hipError_t launch_prefill_t(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *init, const int32_t *cu,
                                   int32_t N, int32_t T_tot, int32_t H, int32_t dv, void *out,
                                   float *fin, hipStream_t stream)
{
    typedef PrefillCfg<TIn, C, NW> P;
    auto kern = kda_prefill_kernel<TIn, C, NW>;
    static bool attr_set = false;   // idempotent; racing threads set the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)P::bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int64_t units = (int64_t)N * H;
    const int nblk = dv / P::BV;
    const int64_t groups = (units + 7) / 8;
    const int64_t grid = groups * 8 * nblk;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(P::NT), P::bytes, stream,
                       static_cast<const TIn *>(q), static_cast<const TIn *>(k), static_cast<const TIn *>(v),
                       g, beta, init, cu, N, T_tot, H, dv, static_cast<TIn *>(out), fin);
    return hipGetLastError();
}

}  // namespace kda

// Dispatch on (dtype, chunk, dv_block); returns hipErrorInvalidValue for an
// unsupported combination (the host API validates before calling).
extern "C" hipError_t kda_launch_prefill(int bf16, int chunk, int dv_block,
                                         const void *q, const void *k, const void *v,
                                         const float *g, const float *beta, const float *init,
                                         const int32_t *cu, int32_t N, int32_t T_tot, int32_t H,
                                         int32_t dv, void *out, float *fin, hipStream_t stream)
{
    using namespace kda;
#define KDA_CASE(TT, CC, NWW)                                                                    \
    if (chunk == CC && dv_block == 16 * NWW)                                                       \
        return launch_prefill_t<TT, CC, NWW>(q, k, v, g, beta, init, cu, N, T_tot, H, dv, out, fin, stream);
    if (bf16) {
        KDA_CASE(bf16_t, 64, 1) KDA_CASE(bf16_t, 64, 2) KDA_CASE(bf16_t, 64, 4) KDA_CASE(bf16_t, 64, 8)
        KDA_CASE(bf16_t, 32, 1) KDA_CASE(bf16_t, 32, 2) KDA_CASE(bf16_t, 32, 4) KDA_CASE(bf16_t, 32, 8)
    } else {
        KDA_CASE(float, 32, 1) KDA_CASE(float, 32, 2) KDA_CASE(float, 32, 4) KDA_CASE(float, 32, 8)
        KDA_CASE(float, 16, 1) KDA_CASE(float, 16, 2) KDA_CASE(float, 16, 4) KDA_CASE(float, 16, 8)
    }
#undef KDA_CASE
    return hipErrorInvalidValue;
}
