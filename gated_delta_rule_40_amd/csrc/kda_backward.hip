// kda_backward.hip -- gradients of the KDA recurrence (training), chunk form.
//
// The recurrence (page ailearn.mscapital.top/kimi-k3.html, card "KDA 单头递归"),
// S_t = (I - b_t k_t k_t^T) Diag(e^g_t) S_{t-1} + b_t k_t v_t^T, o_t = S_t^T q_t,
// runs forward in the chunk form of kda_prefill.hip.  Its gradients come in
// three steps, all chunk-parallel or segment-parallel:
//   1. the forward pipeline stores the state at every chunk start (and the
//      chunk-operand pass writes, next to each chunk image, the transposed
//      "gradient image");
//   2. the state gradient G_t = dL/dS_t runs backwards through the chunks in
//      chunk form (kda_grad_chain_kernel, kda_prefill.hip): per segment from a
//      zero gradient (summaries), a reverse combine through the transposed
//      forward transitions, then every segment from its entering gradient,
//      storing G at every chunk end;
//   3. kda_bwd_chunk_kernel (below) turns each chunk's S (start), G (end) and
//      inputs into its gradients of q, k, v, g and beta -- no recurrence left,
//      one workgroup per (chunk, head).
#include "kda_device.hpp"

namespace kda {

constexpr int BD = 128;              // dk = dv

__device__ __forceinline__ float dot4(const f32x4 &a, const f32x4 &b) {
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// Sums across lanes: over the 16 lanes of a DPP row (a row of an MFMA tile's
// columns), and over the four DPP rows (the lane groups that share a column).
__device__ __forceinline__ float sum16(float x) {       // over the 16 lanes of each DPP row
    x += dpp_mov<0xB1>(x);                             // quad_perm(1,0,3,2): lane ^ 1
    x += dpp_mov<0x4E>(x);                             // quad_perm(2,3,0,1): lane ^ 2
    x += dpp_mov<0x141>(x);                            // row_half_mirror: lane ^ 7 within 8
    return x + dpp_mov<0x140>(x);                      // row_mirror: lane ^ 15 within 16
}
__device__ __forceinline__ float sum_rows4(float x) {  // over the four DPP rows
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ============================================================ chunk form
// Per (chunk, head) gradients from the state S at the chunk start and the
// state gradient G at its end (fp32, [DK][DK] row-major; S from the forward
// pipeline's chunk-start states, G from the state-gradient chain).  With the
// chunk form of the forward (kda_prefill.hip; chunk of C tokens, Gamma the
// cumulative gate, K+ = K (.) e^Gamma, Q+ = Q (.) e^Gamma, K^ = K (.)
// e^(Gamma_L - Gamma), A, P the decayed Gram tiles, N = Diag(b) A,
// T = (I + N)^-1, E_ric = e^(Gamma_rc - Gamma_ic)), the chain rule gives
//     U = V - K+ S,   X = Diag(b) U,   W = T X
//     dW = K^ G + P^T dO,   dX = T^T dW,   dv = Diag(b) dX
//     dQ+ = dO S^T,   dK+ = -Diag(b) dX S^T,   dK^ = W G^T
//     dP = tril(dO W^T),   dN = -stril(dX W^T),   dA = Diag(b) dN
//     dbeta_r = sum_i dN_ri A_ri + sum_c U_rc dX_rc
//     dq = dQ+ (.) e^Gamma + sum_i dP_ri k_i (.) E_ri
//     dk = dK+ (.) e^Gamma + sum_i dA_ri k_i (.) E_ri                      (row part)
//        + dK^ (.) e^(Gamma_L - Gamma) + sum_r (dA_ri k_r + dP_ri q_r) (.) E_ri   (column part)
//     dGamma = q (.) dq + k (.) (row part) - k (.) (column part), and at the
//              last token also sum_r k (.) dK^ (.) e^(Gamma_L - Gamma) + (G (.) S) 1 (.) e^Gamma_L
//     dg = reverse cumulative sum of dGamma over the chunk.
// Everything runs on fp32 (MFMA 16x16x4 and VALU), for both input types.
// Gamma is kept in fp64: every decay factor is e^x of a difference of two of
// its entries, rounded to fp32 only then, so a factor carries the rounding of
// its own exponent, not that of the (up to 160 in magnitude) cumulative sums.
// E is factored per 16-token block pair with a reference inside the pair --
// the middle token of a diagonal block, the block boundary for the
// off-diagonal one -- so every factor lies in [e^-80, e^40] for g in [-5, 0]:
// the Gram tiles and the E-weighted token sums are then plain MFMA products of
// factored operands, and a factor applied after a product is at most e^40.
namespace bc {
constexpr int C = 32, NT = 256;
constexpr int LDG = BD + 2;          // fp64 Gamma rows
constexpr int LDF = BD + 4;          // fp32 [C][BD] rows
constexpr int LDX = C + 4;           // fp32 [C][C] rows
template <typename T>
struct Cfg {
    static constexpr int LDI = BD + 16 / (int)sizeof(T);   // q, k rows (input type)
    static constexpr uint32_t offK = 0;
    static constexpr uint32_t offQ = offK + sizeof(T) * C * LDI;
    static constexpr uint32_t offGm = (offQ + sizeof(T) * C * LDI + 15) / 16 * 16;
    static constexpr uint32_t offDO = offGm + sizeof(double) * C * LDG;
    static constexpr uint32_t offW = offDO + sizeof(float) * C * LDF;     // W, later dGamma
    static constexpr uint32_t offDX = offW + sizeof(float) * C * LDF;
    static constexpr uint32_t offA = offDX + sizeof(float) * C * LDF;
    static constexpr uint32_t offP = offA + sizeof(float) * C * LDX;      // P, later dP
    static constexpr uint32_t offPT = offP + sizeof(float) * C * LDX;     // P^T, later dP^T
    static constexpr uint32_t offT = offPT + sizeof(float) * C * LDX;     // T, later dA
    static constexpr uint32_t offTT = offT + sizeof(float) * C * LDX;     // T^T, later dA^T
    static constexpr uint32_t offBeta = offTT + sizeof(float) * C * LDX;
    static constexpr uint32_t offDb = offBeta + sizeof(float) * C;        // [8][C] partial dbeta
    static constexpr uint32_t bytes = offDb + sizeof(float) * 8 * C;
    static_assert(bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};
typedef double f64x2 __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ f32x4 ld4(const T *p);
template <> __device__ __forceinline__ f32x4 ld4<float>(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
template <> __device__ __forceinline__ f32x4 ld4<bf16_t>(const bf16_t *p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{to_f(x[0]), to_f(x[1]), to_f(x[2]), to_f(x[3])};
}
// e^(a_e - b_e) for four consecutive fp64 entries, the differences in fp64
__device__ __forceinline__ f32x4 exp_diff4(const double *a, const double *b) {
    const f64x2 a0 = *reinterpret_cast<const f64x2 *>(a), a1 = *reinterpret_cast<const f64x2 *>(a + 2);
    const f64x2 b0 = *reinterpret_cast<const f64x2 *>(b), b1 = *reinterpret_cast<const f64x2 *>(b + 2);
    return f32x4{__expf((float)(a0[0] - b0[0])), __expf((float)(a0[1] - b0[1])), __expf((float)(a1[0] - b1[0])),
                 __expf((float)(a1[1] - b1[1]))};
}
__device__ __forceinline__ f32x4 exp4(const double *a) {
    const f64x2 a0 = *reinterpret_cast<const f64x2 *>(a), a1 = *reinterpret_cast<const f64x2 *>(a + 2);
    return f32x4{__expf((float)a0[0]), __expf((float)a0[1]), __expf((float)a1[0]), __expf((float)a1[1])};
}
}  // namespace bc

template <typename T>
__global__ __launch_bounds__(bc::NT) void kda_bwd_chunk_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ g,
    const float *__restrict__ beta, const T *__restrict__ dout, const float *initial_state,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, const float *__restrict__ snaps,
    const float *__restrict__ gchunk, int32_t N, int32_t T_tot, int32_t H, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dg, float *__restrict__ dbeta)
{
    using namespace bc;
    typedef Cfg<T> Q;
    typedef Mma<float> Mf;
    constexpr int LDI = Q::LDI;
    extern __shared__ __align__(16) unsigned char smem[];
    T *sK = reinterpret_cast<T *>(smem + Q::offK);
    T *sQ = reinterpret_cast<T *>(smem + Q::offQ);
    double *sGm = reinterpret_cast<double *>(smem + Q::offGm);
    float *sDO = reinterpret_cast<float *>(smem + Q::offDO);
    float *sW = reinterpret_cast<float *>(smem + Q::offW);
    float *sDX = reinterpret_cast<float *>(smem + Q::offDX);
    float *sA = reinterpret_cast<float *>(smem + Q::offA);
    float *sP = reinterpret_cast<float *>(smem + Q::offP);
    float *sPT = reinterpret_cast<float *>(smem + Q::offPT);
    float *sT = reinterpret_cast<float *>(smem + Q::offT);
    float *sTT = reinterpret_cast<float *>(smem + Q::offTT);
    float *sBeta = reinterpret_cast<float *>(smem + Q::offBeta);
    float *sDb = reinterpret_cast<float *>(smem + Q::offDb);
    float *sdP = sP, *sdPT = sPT, *sdA = sT, *sdAT = sTT, *sDG = sW;

    // ---- workgroup -> (chunk, head); the chunk's sequence by binary search
    const int64_t gc = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    if (N <= 0 || gc >= chunk_off[N]) return;
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= gc) lo = mid;
        else hi = mid - 1;
    }
    const int n = lo;
    const int t0 = min(max(cu[n], 0), T_tot), t1 = min(max(cu[n + 1], t0), T_tot);
    const int64_t cs = gc - chunk_off[n];                 // chunk index within the sequence
    const int64_t c0l = t0 + cs * C;
    if (c0l >= t1) return;                                // only when cu_seqlens is not non-decreasing
    const int c0 = (int)c0l, L = min(C, t1 - c0);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane >> 4, lm = lane & 15;
    const int64_t rowQ = (int64_t)H * BD;
    const int64_t hoff = (int64_t)h * BD;
    const float *Sg = cs ? snaps + (gc * H + h) * BD * BD
                         : (initial_state ? initial_state + ((int64_t)n * H + h) * BD * BD : nullptr);
    const float *Gg = gchunk + (gc * H + h) * BD * BD;

    // ---- 0. the chunk's q, k (input type), dO (fp32), beta and Gamma (fp64);
    //         rows past the chunk's end are zero (Gamma stays constant)
    {
        constexpr int VE = 16 / (int)sizeof(T), VPR = BD / VE;
        for (int e = tid; e < C * VPR; e += NT) {
            const int r = e / VPR, cv = (e % VPR) * VE;
            const int64_t off = (int64_t)(c0 + min(r, L - 1)) * rowQ + hoff + cv;
            f32x4 kv = *reinterpret_cast<const f32x4 *>(k + off), qv = *reinterpret_cast<const f32x4 *>(q + off);
            if (r >= L) kv = qv = zero4();
            *reinterpret_cast<f32x4 *>(sK + r * LDI + cv) = kv;
            *reinterpret_cast<f32x4 *>(sQ + r * LDI + cv) = qv;
        }
        for (int e = tid; e < C * (BD / 4); e += NT) {
            const int r = e / (BD / 4), cv = (e % (BD / 4)) * 4;
            f32x4 d = ld4(dout + (int64_t)(c0 + min(r, L - 1)) * rowQ + hoff + cv);
            if (r >= L) d = zero4();
            *reinterpret_cast<f32x4 *>(sDO + r * LDF + cv) = d;
        }
        if (tid < C) sBeta[tid] = tid < L ? beta[(int64_t)(c0 + tid) * H + h] : 0.f;
        if (tid < BD) {
            float gv[C];
#pragma unroll
            for (int r = 0; r < C; ++r) gv[r] = g[(int64_t)(c0 + min(r, L - 1)) * rowQ + hoff + tid];
            double s = 0.0;
#pragma unroll
            for (int r = 0; r < C; ++r) {
                if (r < L) s += (double)gv[r];
                sGm[r * LDG + tid] = s;
            }
        }
    }
    __syncthreads();

    // ---- 1. Gram tiles A (strictly lower), P (lower incl.): waves 0, 1 the
    //         diagonal blocks (reference: the block's middle token), wave 2 the
    //         off-diagonal block (reference: token 15); wave 3 zeroes the upper block
    if (wave < 3) {
        const int rb = wave == 0 ? 0 : 16, ib = wave == 1 ? 16 : 0, ref = wave == 0 ? 7 : (wave == 1 ? 23 : 15);
        const int r = rb + lm, i = ib + lm;
        f32x4 accA = zero4(), accP = zero4();
#pragma unroll 2
        for (int kb = 0; kb < BD / 16; ++kb) {
            const int c = 16 * kb + 4 * lj;
            const f32x4 rf = exp_diff4(sGm + r * LDG + c, sGm + ref * LDG + c);
            const f32x4 cf = exp_diff4(sGm + ref * LDG + c, sGm + i * LDG + c);
            const f32x4 b = ld4(sK + i * LDI + c) * cf;
            accA = Mf::mma(ld4(sK + r * LDI + c) * rf, b, accA);
            accP = Mf::mma(ld4(sQ + r * LDI + c) * rf, b, accP);
        }
        const bool diag = wave < 2;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int rr = rb + 4 * lj + ii, cc = ib + lm;
            // selects, not products: entries above the diagonal may be inf
            const float a = (!diag || cc < rr) ? accA[ii] : 0.f;
            const float p = (!diag || cc <= rr) ? accP[ii] : 0.f;
            sA[rr * LDX + cc] = a;
            sP[rr * LDX + cc] = p;
            sPT[cc * LDX + rr] = p;
        }
    } else {
        for (int e = lane; e < 256; e += 64) {
            const int rr = e >> 4, cc = 16 + (e & 15);
            sA[rr * LDX + cc] = 0.f;
            sP[rr * LDX + cc] = 0.f;
            sPT[cc * LDX + rr] = 0.f;
        }
    }
    __syncthreads();

    // ---- 1b. T = (I + Diag(b) A)^-1: the diagonal 16x16 blocks by forward
    //          substitution (waves 0, 1: lane lm computes column lm; the four
    //          lane groups repeat it), then T10 = -T11 (Diag(b) A)_10 T00 (wave 0)
    if (wave < 2) {
        const int a0 = 16 * wave, j = lm;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) s += sA[(a0 + r) * LDX + a0 + i] * t[i];
            t[r] = r == j ? 1.f : (r < j ? 0.f : -sBeta[a0 + r] * s);
        }
        if (lj == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sT[(a0 + r) * LDX + a0 + j] = t[r];
                sTT[(a0 + j) * LDX + a0 + r] = t[r];
            }
        }
    } else {
        for (int e = tid - 128; e < 256; e += 128) {
            const int rr = e >> 4, cc = 16 + (e & 15);
            sT[rr * LDX + cc] = 0.f;
            sTT[cc * LDX + rr] = 0.f;
        }
    }
    __syncthreads();
    if (wave == 0) {
        // X = (Diag(b) A)_10 T00: B[i][j] = T00[i][j] = TT[j][i]
        const f32x4 an = ld4(sA + (16 + lm) * LDX + 4 * lj) * sBeta[16 + lm];
        const f32x4 x = Mf::mma(an, ld4(sTT + lm * LDX + 4 * lj), zero4());
        const f32x4 t10 = -Mf::mma(ld4(sT + (16 + lm) * LDX + 16 + 4 * lj), x, zero4());
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            sT[(16 + 4 * lj + ii) * LDX + lm] = t10[ii];
            sTT[lm * LDX + 16 + 4 * lj + ii] = t10[ii];
        }
    }
    __syncthreads();

    // ---- 2. value columns vc0, vc0 + 16 of this wave (tiles ct), token row tiles rt
    const int vc0 = 32 * wave + lm;
    f32x4 U[2][2], dW[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) U[rt][ct] = dW[rt][ct] = zero4();
    const double *gmL = sGm + (L - 1) * LDG;
#pragma unroll 2
    for (int kb = 0; kb < BD / 16; ++kb) {
        const int c = 16 * kb + 4 * lj;
        f32x4 sb[2], gb[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sb[ct][e] = Sg ? Sg[(int64_t)(c + e) * BD + vc0 + 16 * ct] : 0.f;
                gb[ct][e] = Gg[(int64_t)(c + e) * BD + vc0 + 16 * ct];
            }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int r = 16 * rt + lm;
            const f32x4 kr = ld4(sK + r * LDI + c);
            const f32x4 kp = kr * exp4(sGm + r * LDG + c);                 // K+
            const f32x4 kh = kr * exp_diff4(gmL + c, sGm + r * LDG + c);   // K^
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                U[rt][ct] = Mf::mma(kp, sb[ct], U[rt][ct]);
                dW[rt][ct] = Mf::mma(kh, gb[ct], dW[rt][ct]);
            }
        }
    }
    f32x4 X[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * lj + i;
                const float vv = to_f(v[(int64_t)(c0 + min(r, L - 1)) * rowQ + hoff + vc0 + 16 * ct]);
                U[rt][ct][i] = (r < L ? vv : 0.f) - U[rt][ct][i];
                X[rt][ct][i] = sBeta[r] * U[rt][ct][i];
            }
    // W = T X;  dW += P^T dO;  dX = T^T dW   (T lower, P^T and T^T upper by blocks)
    f32x4 W[2][2], dX[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) W[rt][ct] = zero4();
#pragma unroll
        for (int bt = 0; bt <= rt; ++bt) {
            const f32x4 ta = ld4(sT + (16 * rt + lm) * LDX + 16 * bt + 4 * lj);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) W[rt][ct] = Mf::mma(ta, X[bt][ct], W[rt][ct]);
        }
#pragma unroll
        for (int bt = rt; bt < 2; ++bt) {
            const f32x4 pa = ld4(sPT + (16 * rt + lm) * LDX + 16 * bt + 4 * lj);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                f32x4 db;
#pragma unroll
                for (int e = 0; e < 4; ++e) db[e] = sDO[(16 * bt + 4 * lj + e) * LDF + vc0 + 16 * ct];
                dW[rt][ct] = Mf::mma(pa, db, dW[rt][ct]);
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) dX[rt][ct] = zero4();
#pragma unroll
        for (int bt = rt; bt < 2; ++bt) {
            const f32x4 ta = ld4(sTT + (16 * rt + lm) * LDX + 16 * bt + 4 * lj);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) dX[rt][ct] = Mf::mma(ta, dW[bt][ct], dX[rt][ct]);
        }
    }
    // dv, the U.dX part of dbeta (this wave's columns), W and dX to LDS
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * lj + i;
            float pb = 0.f;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int col = vc0 + 16 * ct;
                if (r < L) dv[(int64_t)(c0 + r) * rowQ + hoff + col] = sBeta[r] * dX[rt][ct][i];
                pb += U[rt][ct][i] * dX[rt][ct][i];
                sW[r * LDF + col] = W[rt][ct][i];
                sDX[r * LDF + col] = dX[rt][ct][i];
            }
            pb = sum16(pb);
            if (lm == 0) sDb[wave * C + r] = pb;
        }
    __syncthreads();

    // ---- 3. contractions over the value columns: key channels cc of this
    //         wave (tiles ct), S and G rows read from global memory
    f32x4 dQp[2][2], dXS[2][2], dKh[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) dQp[rt][ct] = dXS[rt][ct] = dKh[rt][ct] = zero4();
    float dgm[2] = {0.f, 0.f};
#pragma unroll 2
    for (int kb = 0; kb < BD / 16; ++kb) {
        const int j = 16 * kb + 4 * lj;
        f32x4 st[2], gt[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int cc = 32 * wave + 16 * ct + lm;
            st[ct] = Sg ? *reinterpret_cast<const f32x4 *>(Sg + (int64_t)cc * BD + j) : zero4();
            gt[ct] = *reinterpret_cast<const f32x4 *>(Gg + (int64_t)cc * BD + j);
            dgm[ct] += dot4(st[ct], gt[ct]);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int r = 16 * rt + lm;
            const f32x4 ado = ld4(sDO + r * LDF + j), adx = ld4(sDX + r * LDF + j), aw = ld4(sW + r * LDF + j);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                dQp[rt][ct] = Mf::mma(ado, st[ct], dQp[rt][ct]);
                dXS[rt][ct] = Mf::mma(adx, st[ct], dXS[rt][ct]);
                dKh[rt][ct] = Mf::mma(aw, gt[ct], dKh[rt][ct]);
            }
        }
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) dgm[ct] = sum_rows4(dgm[ct]);   // (G (.) S) 1 of channel cc
    // dP and dN: waves 0, 1 the diagonal blocks, wave 2 the off-diagonal one
    // (they overwrite P, P^T, T, T^T, whose last reads were in part 2)
    if (wave < 3) {
        const int rb = wave == 0 ? 0 : 16, ib = wave == 1 ? 16 : 0;
        const bool diag = wave < 2;
        f32x4 accP = zero4(), accN = zero4();
#pragma unroll 2
        for (int kb = 0; kb < BD / 16; ++kb) {
            const int j = 16 * kb + 4 * lj;
            const f32x4 bw = ld4(sW + (ib + lm) * LDF + j);
            accP = Mf::mma(ld4(sDO + (rb + lm) * LDF + j), bw, accP);
            accN = Mf::mma(ld4(sDX + (rb + lm) * LDF + j), bw, accN);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int rr = rb + 4 * lj + ii, cc = ib + lm;
            const float dp = (!diag || cc <= rr) ? accP[ii] : 0.f;
            const float dn = (!diag || cc < rr) ? -accN[ii] : 0.f;
            const float da = sBeta[rr] * dn;
            sdP[rr * LDX + cc] = dp;
            sdPT[cc * LDX + rr] = dp;
            sdA[rr * LDX + cc] = da;
            sdAT[cc * LDX + rr] = da;
            const float pb = sum16(dn * sA[rr * LDX + cc]);
            if (lm == 0) sDb[(4 + wave) * C + rr] = pb;
        }
    } else {
        for (int e = lane; e < 256; e += 64) {
            const int rr = e >> 4, cc = 16 + (e & 15);
            sdP[rr * LDX + cc] = 0.f;
            sdPT[cc * LDX + rr] = 0.f;
            sdA[rr * LDX + cc] = 0.f;
            sdAT[cc * LDX + rr] = 0.f;
        }
        if (lane < 16) {      // rows that a block's dbeta part does not cover
            sDb[4 * C + 16 + lane] = 0.f;
            sDb[5 * C + lane] = 0.f;
            sDb[6 * C + lane] = 0.f;
            sDb[7 * C + lane] = 0.f;
            sDb[7 * C + 16 + lane] = 0.f;
        }
    }
    __syncthreads();

    // ---- 4. token sums weighted by E, and the per-element results
#pragma unroll 1
    for (int ct = 0; ct < 2; ++ct) {
        const int c = 32 * wave + 16 * ct + lm;
        auto gm = [&](int t) { return sGm[t * LDG + c]; };
        auto kv = [&](int t) { return to_f(sK[t * LDI + c]); };
        auto qv = [&](int t) { return to_f(sQ[t * LDI + c]); };
        // B operands over tokens: lane group lj takes tokens tb + 4 lj + e
        f32x4 Kcd[2], Krd[2], Qrd[2], Kco, Kro, Qro;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const double gmid = gm(16 * a + 7);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * a + 4 * lj + e;
                const float d = (float)(gm(t) - gmid);
                const float rf = __expf(d);
                Kcd[a][e] = kv(t) * __expf(-d);
                Krd[a][e] = kv(t) * rf;
                Qrd[a][e] = qv(t) * rf;
            }
        }
        const double g15 = gm(15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t0_ = 4 * lj + e, t1_ = 16 + 4 * lj + e;
            Kco[e] = kv(t0_) * __expf((float)(g15 - gm(t0_)));
            const float ro = __expf((float)(gm(t1_) - g15));
            Kro[e] = kv(t1_) * ro;
            Qro[e] = qv(t1_) * ro;
        }
        f32x4 q2d[2], kr2d[2], kc2d[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int ro = (16 * a + lm) * LDX + 16 * a + 4 * lj;
            q2d[a] = Mf::mma(ld4(sdP + ro), Kcd[a], zero4());
            kr2d[a] = Mf::mma(ld4(sdA + ro), Kcd[a], zero4());
            kc2d[a] = Mf::mma(ld4(sdAT + ro), Krd[a], Mf::mma(ld4(sdPT + ro), Qrd[a], zero4()));
        }
        const f32x4 q2o = Mf::mma(ld4(sdP + (16 + lm) * LDX + 4 * lj), Kco, zero4());
        const f32x4 kr2o = Mf::mma(ld4(sdA + (16 + lm) * LDX + 4 * lj), Kco, zero4());
        const f32x4 kc2o = Mf::mma(ld4(sdAT + lm * LDX + 16 + 4 * lj), Kro,
                                   Mf::mma(ld4(sdPT + lm * LDX + 16 + 4 * lj), Qro, zero4()));
        // the last token's extra terms: sum_r k dK^ e^(Gamma_L - Gamma) and (G (.) S) 1 e^Gamma_L
        const double gl = gm(L - 1);
        float extra = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int r = 16 * rt + 4 * lj + ii;
                extra += kv(r) * dKh[rt][ct][ii] * __expf((float)(gl - gm(r)));
            }
        extra = sum_rows4(extra) + dgm[ct] * __expf((float)gl);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int r = 16 * rt + 4 * lj + ii;
                const double gr = gm(r), gmid = gm(16 * rt + 7);
                const float dmid = (float)(gr - gmid);
                float dq2 = __expf(dmid) * q2d[rt][ii], dkr2 = __expf(dmid) * kr2d[rt][ii];
                float dkc2 = __expf(-dmid) * kc2d[rt][ii];
                if (rt == 1) {
                    const float ro = __expf((float)(gr - g15));
                    dq2 += ro * q2o[ii];
                    dkr2 += ro * kr2o[ii];
                } else {
                    dkc2 += __expf((float)(g15 - gr)) * kc2o[ii];
                }
                const float eG = __expf((float)gr), eGn = __expf((float)(gl - gr));
                const float dq_ = dQp[rt][ct][ii] * eG + dq2;
                const float dkrow = -sBeta[r] * dXS[rt][ct][ii] * eG + dkr2;
                const float dkcol = dKh[rt][ct][ii] * eGn + dkc2;
                const float kr = kv(r);
                float dG = qv(r) * dq_ + kr * dkrow - kr * dkcol;
                if (r == L - 1) dG += extra;
                if (r < L) {
                    dq[(int64_t)(c0 + r) * rowQ + hoff + c] = dq_;
                    dk[(int64_t)(c0 + r) * rowQ + hoff + c] = dkrow + dkcol;
                }
                sDG[r * LDF + c] = dG;
            }
    }
    __syncthreads();

    // ---- 5. dg = reverse cumulative sum of dGamma; dbeta from its parts
    if (tid < BD) {
        float acc = 0.f;
        for (int r = L - 1; r >= 0; --r) {
            acc += sDG[r * LDF + tid];
            dg[(int64_t)(c0 + r) * rowQ + hoff + tid] = acc;
        }
    } else if (tid < BD + C) {
        const int r = tid - BD;
        if (r < L) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) s += sDb[w * C + r];
            dbeta[(int64_t)(c0 + r) * H + h] = s;
        }
    }
}

}  // namespace kda

// Per (chunk, head) gradients of the chunk form (kda_bwd_chunk_kernel): S at
// every chunk start in snaps (a sequence's first chunk: initial_state, or zero
// if nullptr), the gradient at every chunk end in gchunk, both [chunks][H][BD][BD].
extern "C" hipError_t kda_launch_bwd_chunk(int bf16, const void *q, const void *k, const void *v, const float *g,
                                           const float *beta, const void *dout, const float *init, const int32_t *cu,
                                           const int32_t *chunk_off, int64_t max_chunks, const float *snaps,
                                           const float *gchunk, int32_t N, int32_t T_tot, int32_t H, float *dq,
                                           float *dk, float *dv, float *dg, float *dbeta, hipStream_t stream)
{
    using namespace kda;
    const int64_t grid = max_chunks * H;
    if (grid <= 0 || N <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (bf16) {
        auto kern = kda_bwd_chunk_kernel<bf16_t>;
        static std::atomic<uint64_t> lds_set{0};
        if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(kern), (int)bc::Cfg<bf16_t>::bytes, lds_set))
            return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(bc::NT), bc::Cfg<bf16_t>::bytes, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k),
                           static_cast<const bf16_t *>(v), g, beta, static_cast<const bf16_t *>(dout), init, cu,
                           chunk_off, snaps, gchunk, N, T_tot, H, dq, dk, dv, dg, dbeta);
    } else {
        auto kern = kda_bwd_chunk_kernel<float>;
        static std::atomic<uint64_t> lds_set{0};
        if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(kern), (int)bc::Cfg<float>::bytes, lds_set))
            return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(bc::NT), bc::Cfg<float>::bytes, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(v), g, beta, static_cast<const float *>(dout), init, cu,
                           chunk_off, snaps, gchunk, N, T_tot, H, dq, dk, dv, dg, dbeta);
    }
    return hipGetLastError();
}
