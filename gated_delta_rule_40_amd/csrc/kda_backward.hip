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
#include <type_traits>

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
// state gradient G at its end, with the chunk form of the forward
// (kda_prefill.hip; chunk of C tokens, Gamma the cumulative gate, K+ = K (.)
// e^Gamma, Q+ = Q (.) e^Gamma, K^ = K (.) e^(Gamma_L - Gamma), A, P the decayed
// Gram tiles, N = Diag(b) A, E_ric = e^(Gamma_rc - Gamma_ic)).  The chain rule
// gives, with U = V - K+ S, W = (I + N)^-1 Diag(b) U (the forward's) and
// dX = (I + N)^-T (K^ G + P^T dO) (the state-gradient chain's; dv = Diag(b) dX):
//     dQ+ = dO S^T,   dK+ = -Diag(b) dX S^T,   dK^ = W G^T
//     dP = tril(dO W^T),   dN = -stril(dX W^T),   dA = Diag(b) dN
//     dbeta_r = sum_i dN_ri A_ri + sum_c U_rc dX_rc
//     dq = dQ+ (.) e^Gamma + sum_i dP_ri k_i (.) E_ri
//     dk = dK+ (.) e^Gamma + sum_i dA_ri k_i (.) E_ri                      (row part)
//        + dK^ (.) e^(Gamma_L - Gamma) + sum_r (dA_ri k_r + dP_ri q_r) (.) E_ri   (column part)
//     dGamma = q (.) dq + k (.) (row part) - k (.) (column part), and at the
//              last token also sum_r k (.) dK^ (.) e^(Gamma_L - Gamma) + (G (.) S) 1 (.) e^Gamma_L
//     dg = reverse cumulative sum of dGamma over the chunk.
// U and W come from the forward pass that stores the chunk-start states, dX
// from the state-gradient chain (which also writes dv), S and G as those
// passes store them.  What is left here has no recurrence: one workgroup per
// (chunk, head).
// Precision: the Gram tile A and every 32-wide contraction run on fp32 (MFMA
// 16x16x4 and VALU).  The five 128-wide contractions (dQ+, dX S^T, dK^, dP,
// dN) run on the MFMA type of the forward: fp32 for fp32 inputs; fp16 for
// 16-bit inputs, with S and G read as the fp16 values and exact power-of-two
// column scales that the chains carry, and every other operand given an exact
// power-of-two scale per row (the row maximum lands in [2^13, 2^14)) -- a
// scale along the contraction index is folded into the other operand, so every
// product is exact up to the fp16 rounding of its operands.
// Gamma is kept in fp64: every decay factor is e^x of a difference of two of
// its entries, rounded to fp32 only then, so a factor carries the rounding of
// its own exponent, not that of the (up to 160 in magnitude) cumulative sums.
// E is factored per 16-token block pair with a reference inside the pair --
// the middle token of a diagonal block, the block boundary for the
// off-diagonal one -- so every factor lies in [e^-80, e^40] for g in [-5, 0]:
// the Gram tile and the E-weighted token sums are then plain MFMA products of
// factored operands, and a factor applied after a product is at most e^40.
// Work split: eight waves; in the key-channel parts wave w owns channels
// 16 w .. 16 w + 15; token rows are loaded by 16 lanes each (8 columns per lane).
namespace bc {
constexpr int C = 32, NW = 8, NT = 64 * NW;
constexpr int LDG = BD + 2;          // fp64 Gamma rows
constexpr int LDF = BD + 4;          // fp32 [C][BD] rows
constexpr int LDX = C + 4;           // fp32 [C][C] rows
constexpr int NDB = 4;               // partial dbeta slots: U.dX, and the dN (.) A part of 3 blocks
constexpr int NMX = 6;               // row scales from |dO|, |dO|/sS, |dX|, |dX|/sS, |W|, |W|/sG
enum { MX_DO = 0, MX_DOS = 1, MX_DX = 2, MX_DXS = 3, MX_W = 4, MX_WG = 5 };
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
    static constexpr uint32_t offdP = offA + sizeof(float) * C * LDX;
    static constexpr uint32_t offdPT = offdP + sizeof(float) * C * LDX;
    static constexpr uint32_t offdA = offdPT + sizeof(float) * C * LDX;
    static constexpr uint32_t offdAT = offdA + sizeof(float) * C * LDX;
    static constexpr uint32_t offGp = offdAT + sizeof(float) * C * LDX;   // [3][256] partial Gram tiles
    static constexpr uint32_t offBeta = offGp + sizeof(float) * 3 * 256;
    static constexpr uint32_t offDb = offBeta + sizeof(float) * C;        // [NDB][C] partial dbeta
    static constexpr uint32_t offIS = offDb + sizeof(float) * NDB * C;    // [BD] 1 / column scale of S
    static constexpr uint32_t offIG = offIS + sizeof(float) * BD;         // [BD] 1 / column scale of G
    static constexpr uint32_t offRS = offIG + sizeof(float) * BD;         // [NMX][C] row scales
    static constexpr uint32_t bytes = offRS + sizeof(float) * NMX * C;
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
__device__ __forceinline__ float max4(const f32x4 &x) { return fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])); }
__device__ __forceinline__ f32x4 abs4(const f32x4 &x) { return f32x4{fabsf(x[0]), fabsf(x[1]), fabsf(x[2]), fabsf(x[3])}; }
// Contraction indices of element e of lane group j's K-block fragment, in
// groups of four consecutive ones: group 0 at k0 + 4 j, and for 16-bit
// operands group 1 at k0 + 16 + 4 j (the layout of kda_device.hpp).
template <typename OpT> struct Frag {
    typedef Mma<OpT> M;
    static constexpr int NG = M::KB / 16;                 // groups of four per fragment
    __device__ static __forceinline__ int base(int k0, int j, int gi) { return k0 + 16 * gi + 4 * j; }
    // fragment from NG f32x4 groups, each element times `scale`
    __device__ static __forceinline__ typename M::frag make(const f32x4 (&x)[NG], float scale) {
        typename M::frag f;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int e = 0; e < 4; ++e) f[4 * gi + e] = from_f<OpT>(x[gi][e] * scale);
        return f;
    }
};
}  // namespace bc

// S (start state) and G (end gradient) of every chunk: [chunks][H][BD][BD] as
// the chains store them -- fp16 values with column scales [chunks][H][BD]
// (OpT = fp16) or fp32 (scales unused); U, W, dX: [chunks][H][C][BD] fp32.
template <typename T>
__global__ __launch_bounds__(bc::NT) void kda_bwd_chunk_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const T *__restrict__ dout, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const void *__restrict__ snaps, const float *__restrict__ snap_scale,
    const void *__restrict__ gchunk, const float *__restrict__ g_scale, const float *__restrict__ uw_u,
    const float *__restrict__ uw_w, const float *__restrict__ dx_chunk, int32_t N, int32_t T_tot, int32_t H,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dg,
    float *__restrict__ dbeta)
{
    using namespace bc;
    typedef Cfg<T> Q;
    typedef Mma<float> Mf;
    constexpr bool kIn16 = !std::is_same<T, float>::value;
    typedef typename std::conditional<kIn16, f16_t, float>::type OpT;   // 128-wide contractions
    typedef Mma<OpT> Mo;
    typedef Frag<OpT> F;
    constexpr int KB = Mo::KB, NG = F::NG;
    constexpr int LDI = Q::LDI;
    extern __shared__ __align__(16) unsigned char smem[];
    T *sK = reinterpret_cast<T *>(smem + Q::offK);
    T *sQ = reinterpret_cast<T *>(smem + Q::offQ);
    double *sGm = reinterpret_cast<double *>(smem + Q::offGm);
    float *sDO = reinterpret_cast<float *>(smem + Q::offDO);
    float *sW = reinterpret_cast<float *>(smem + Q::offW);
    float *sDX = reinterpret_cast<float *>(smem + Q::offDX);
    float *sA = reinterpret_cast<float *>(smem + Q::offA);
    float *sdP = reinterpret_cast<float *>(smem + Q::offdP);
    float *sdPT = reinterpret_cast<float *>(smem + Q::offdPT);
    float *sdA = reinterpret_cast<float *>(smem + Q::offdA);
    float *sdAT = reinterpret_cast<float *>(smem + Q::offdAT);
    float *sGp = reinterpret_cast<float *>(smem + Q::offGp);
    float *sBeta = reinterpret_cast<float *>(smem + Q::offBeta);
    float *sDb = reinterpret_cast<float *>(smem + Q::offDb);
    float *sIS = reinterpret_cast<float *>(smem + Q::offIS);
    float *sIG = reinterpret_cast<float *>(smem + Q::offIG);
    float *sRS = reinterpret_cast<float *>(smem + Q::offRS);
    float *sDG = sW;

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
    const int64_t c0l = t0 + (gc - chunk_off[n]) * C;
    if (c0l >= t1) return;                                // only when cu_seqlens is not non-decreasing
    const int c0 = (int)c0l, L = min(C, t1 - c0);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane >> 4, lm = lane & 15;
    const int64_t rowQ = (int64_t)H * BD;
    const int64_t hoff = (int64_t)h * BD;
    const int64_t unit = gc * H + h;
    const OpT *Sg = static_cast<const OpT *>(snaps) + unit * BD * BD;
    const OpT *Gg = static_cast<const OpT *>(gchunk) + unit * BD * BD;
    // S and G rows of this lane's key channel for part 3, loaded now so that
    // they arrive during parts 0-1 (fragment order: K-block, group)
    typedef typename std::conditional<kIn16, f16x4, f32x4>::type V4;
    const int cc = 16 * wave + lm;
    V4 spre[BD / KB][NG], gpre[BD / KB][NG];
#pragma unroll
    for (int kb = 0; kb < BD / KB; ++kb)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int j = F::base(kb * KB, lj, gi);
            spre[kb][gi] = *reinterpret_cast<const V4 *>(Sg + (int64_t)cc * BD + j);
            gpre[kb][gi] = *reinterpret_cast<const V4 *>(Gg + (int64_t)cc * BD + j);
        }
    asm volatile("" ::: "memory");                        // keeps the loads here

    // ---- 0. loads.  Thread (row r = tid / 16, part m = tid % 16) takes columns
    //         8 m .. 8 m + 7 of row r of q, k, dO, W, dX (and U, for the U.dX
    //         part of dbeta, and the column scales of S and G); a row's 16
    //         parts are one DPP row, so its sums and maxima are taken across
    //         those lanes.  Threads 0-127 also take channel tid of the gate for
    //         the fp64 cumulative sum.  Every global load is issued first, so
    //         that the part waits for memory once.
    {
        typedef typename std::conditional<kIn16, f32x4, f32x4[2]>::type Raw8;   // 8 input elements
        const int r = tid >> 4, m = tid & 15, cb = 8 * m;
        const bool ok = r < L;
        const int64_t off = (int64_t)(c0 + min(r, L - 1)) * rowQ + hoff + cb;
        const int64_t cho = unit * C * BD + (int64_t)r * BD + cb;   // (chunk, head) row r of U, W, dX
        Raw8 kraw, qraw, draw;
        if constexpr (kIn16) {
            kraw = *reinterpret_cast<const f32x4 *>(k + off);
            qraw = *reinterpret_cast<const f32x4 *>(q + off);
            draw = *reinterpret_cast<const f32x4 *>(dout + off);
        } else {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                kraw[hf] = *reinterpret_cast<const f32x4 *>(k + off + 4 * hf);
                qraw[hf] = *reinterpret_cast<const f32x4 *>(q + off + 4 * hf);
                draw[hf] = *reinterpret_cast<const f32x4 *>(dout + off + 4 * hf);
            }
        }
        f32x4 w[2], x[2], u[2], ss[2], sg[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {   // rows past the chunk read row r of the block (stored, not used)
            w[hf] = *reinterpret_cast<const f32x4 *>(uw_w + cho + 4 * hf);
            x[hf] = *reinterpret_cast<const f32x4 *>(dx_chunk + cho + 4 * hf);
            u[hf] = *reinterpret_cast<const f32x4 *>(uw_u + cho + 4 * hf);
            ss[hf] = kIn16 ? *reinterpret_cast<const f32x4 *>(snap_scale + unit * BD + cb + 4 * hf) : f32x4{1.f, 1.f, 1.f, 1.f};
            sg[hf] = kIn16 ? *reinterpret_cast<const f32x4 *>(g_scale + unit * BD + cb + 4 * hf) : f32x4{1.f, 1.f, 1.f, 1.f};
        }
        const float br = beta[(int64_t)(c0 + min(r, L - 1)) * H + h];
        float gv[C];
        if (tid < BD) {
#pragma unroll
            for (int i = 0; i < C; ++i) gv[i] = g[(int64_t)(c0 + min(i, L - 1)) * rowQ + hoff + tid];
        }
        asm volatile("" ::: "memory");                    // keeps the loads together
        // q, k as they are (zero past the chunk)
        if constexpr (kIn16) {
            *reinterpret_cast<f32x4 *>(sK + r * LDI + cb) = ok ? kraw : zero4();
            *reinterpret_cast<f32x4 *>(sQ + r * LDI + cb) = ok ? qraw : zero4();
        } else {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                *reinterpret_cast<f32x4 *>(sK + r * LDI + cb + 4 * hf) = ok ? kraw[hf] : zero4();
                *reinterpret_cast<f32x4 *>(sQ + r * LDI + cb + 4 * hf) = ok ? qraw[hf] : zero4();
            }
        }
        f32x4 d[2];
        if constexpr (kIn16) {
            const bf16_t *db = reinterpret_cast<const bf16_t *>(&draw);
            d[0] = ld4(db);
            d[1] = ld4(db + 4);
        } else {
            d[0] = draw[0];
            d[1] = draw[1];
        }
        float ux = 0.f, mx[NMX] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            if (!ok) d[hf] = w[hf] = x[hf] = u[hf] = zero4();
            *reinterpret_cast<f32x4 *>(sDO + r * LDF + cb + 4 * hf) = d[hf];
            *reinterpret_cast<f32x4 *>(sW + r * LDF + cb + 4 * hf) = w[hf];
            *reinterpret_cast<f32x4 *>(sDX + r * LDF + cb + 4 * hf) = x[hf];
            f32x4 is, ig;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                is[e] = pow2_inv(ss[hf][e]);
                ig[e] = pow2_inv(sg[hf][e]);
            }
            if (r == 0) {
                *reinterpret_cast<f32x4 *>(sIS + cb + 4 * hf) = is;
                *reinterpret_cast<f32x4 *>(sIG + cb + 4 * hf) = ig;
            }
            ux += dot4(u[hf], x[hf]);
            mx[MX_DO] = fmaxf(mx[MX_DO], max4(abs4(d[hf])));
            mx[MX_DOS] = fmaxf(mx[MX_DOS], max4(abs4(d[hf]) * is));
            mx[MX_DX] = fmaxf(mx[MX_DX], max4(abs4(x[hf])));
            mx[MX_DXS] = fmaxf(mx[MX_DXS], max4(abs4(x[hf]) * is));
            mx[MX_W] = fmaxf(mx[MX_W], max4(abs4(w[hf])));
            mx[MX_WG] = fmaxf(mx[MX_WG], max4(abs4(w[hf]) * ig));
        }
        if (ok) {                                         // dv = Diag(b) dX
            *reinterpret_cast<f32x4 *>(dv + off) = x[0] * br;
            *reinterpret_cast<f32x4 *>(dv + off + 4) = x[1] * br;
        }
        ux = sum16(ux);
#pragma unroll
        for (int a = 0; a < NMX; ++a) mx[a] = rowmax16(mx[a]);
        if (m == 0) {
            sDb[r] = ux;
            sBeta[r] = ok ? br : 0.f;
#pragma unroll
            for (int a = 0; a < NMX; ++a) sRS[a * C + r] = kIn16 ? pow2_scale(mx[a]) : 1.f;
        }
        if (tid < BD) {
            double sum = 0.0;
#pragma unroll
            for (int i = 0; i < C; ++i) {
                if (i < L) sum += (double)gv[i];
                sGm[i * LDG + tid] = sum;
            }
        }
    }
    __syncthreads();

    // ---- 1. Gram tile A (strictly lower), block x = 0, 1 diagonal (reference:
    //         the block's middle token), x = 2 the off-diagonal one (reference:
    //         token 15); waves x and x + 3 take the two halves of the channels,
    //         wave 6 zeroes the upper block
    f32x4 gacc = zero4();
    const int gx = wave % 3, ghalf = wave / 3;
    const int grb = gx == 0 ? 0 : 16, gib = gx == 1 ? 16 : 0;
    if (wave < 6) {
        const int ref = gx == 0 ? 7 : (gx == 1 ? 23 : 15);
        const int r = grb + lm, i = gib + lm;
#pragma unroll
        for (int kb = 4 * ghalf; kb < 4 * ghalf + 4; ++kb) {
            const int c = 16 * kb + 4 * lj;
            const f32x4 rf = exp_diff4(sGm + r * LDG + c, sGm + ref * LDG + c);
            const f32x4 cf = exp_diff4(sGm + ref * LDG + c, sGm + i * LDG + c);
            gacc = Mf::mma(ld4(sK + r * LDI + c) * rf, ld4(sK + i * LDI + c) * cf, gacc);
        }
        if (ghalf) *reinterpret_cast<f32x4 *>(sGp + gx * 256 + 4 * lane) = gacc;
    } else if (wave == 6) {
        for (int e = lane; e < 256; e += 64) sA[(e >> 4) * LDX + 16 + (e & 15)] = 0.f;
    }
    __syncthreads();
    if (wave < 3) {
        gacc += *reinterpret_cast<const f32x4 *>(sGp + gx * 256 + 4 * lane);
        const bool diag = gx < 2;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int rr = grb + 4 * lj + ii, cc = gib + lm;
            sA[rr * LDX + cc] = (!diag || cc < rr) ? gacc[ii] : 0.f;   // a select: entries above may be inf
        }
    }
    __syncthreads();

    // ---- 3. contractions over the value columns, on the MFMA type of the
    //         forward: key channel cc of this lane (wave w: 16 w + lm); S and G
    //         rows as prefetched (the fragment's indices along the row)
    f32x4 dQp[2], dXS[2], dKh[2];
    dQp[0] = dQp[1] = dXS[0] = dXS[1] = dKh[0] = dKh[1] = zero4();
    float dgm = 0.f;
    const float *rsDOS = sRS + MX_DOS * C, *rsDXS = sRS + MX_DXS * C, *rsWG = sRS + MX_WG * C;
#pragma unroll
    for (int kb = 0; kb < BD / KB; ++kb) {
        typename Mo::frag st, gt;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int j = F::base(kb * KB, lj, gi);
            const V4 sv = spre[kb][gi], gvv = gpre[kb][gi];
            const f32x4 isv = ld4(sIS + j), igv = ld4(sIG + j);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                st[4 * gi + e] = sv[e];
                gt[4 * gi + e] = gvv[e];
                dgm += (float)sv[e] * isv[e] * ((float)gvv[e] * igv[e]);
            }
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int r = 16 * rt + lm;
            f32x4 ado[NG], adx[NG], aw[NG];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int j = F::base(kb * KB, lj, gi);
                const f32x4 isv = ld4(sIS + j), igv = ld4(sIG + j);
                ado[gi] = ld4(sDO + r * LDF + j) * isv;
                adx[gi] = ld4(sDX + r * LDF + j) * isv;
                aw[gi] = ld4(sW + r * LDF + j) * igv;
            }
            dQp[rt] = Mo::mma(F::make(ado, rsDOS[r]), st, dQp[rt]);
            dXS[rt] = Mo::mma(F::make(adx, rsDXS[r]), st, dXS[rt]);
            dKh[rt] = Mo::mma(F::make(aw, rsWG[r]), gt, dKh[rt]);
        }
    }
    dgm = sum_rows4(dgm);                                 // (G (.) S) 1 of channel cc
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {                     // undo the row scales
            const int r = 16 * rt + 4 * lj + i;
            dQp[rt][i] *= pow2_inv(rsDOS[r]);
            dXS[rt][i] *= pow2_inv(rsDXS[r]);
            dKh[rt][i] *= pow2_inv(rsWG[r]);
        }
    // dP (waves 0-2) and dN (waves 3-5) by block x, B = W rows with their own
    // row scales; waves 6-7 zero the upper blocks
    if (wave < 6) {
        const int x = wave % 3;
        const bool isN = wave >= 3, diag = x < 2;
        const int rb = x == 0 ? 0 : 16, ib = x == 1 ? 16 : 0;
        const float *rowA = (isN ? sDX : sDO) + (rb + lm) * LDF;
        const float ra = sRS[(isN ? MX_DX : MX_DO) * C + rb + lm], rw = sRS[MX_W * C + ib + lm];
        f32x4 acc = zero4();
#pragma unroll 2
        for (int kb = 0; kb < BD / KB; ++kb) {
            f32x4 a[NG], b[NG];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int j = F::base(kb * KB, lj, gi);
                a[gi] = ld4(rowA + j);
                b[gi] = ld4(sW + (ib + lm) * LDF + j);
            }
            acc = Mo::mma(F::make(a, ra), F::make(b, rw), acc);
        }
        const float iw = pow2_inv(sRS[MX_W * C + ib + lm]);
        float pb[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int rr = rb + 4 * lj + ii, c2 = ib + lm;
            const float val = acc[ii] * pow2_inv(sRS[(isN ? MX_DX : MX_DO) * C + rr]) * iw;
            if (!isN) {
                const float dp = (!diag || c2 <= rr) ? val : 0.f;
                sdP[rr * LDX + c2] = dp;
                sdPT[c2 * LDX + rr] = dp;
                pb[ii] = 0.f;
            } else {
                const float dn = (!diag || c2 < rr) ? -val : 0.f;
                const float da = sBeta[rr] * dn;
                sdA[rr * LDX + c2] = da;
                sdAT[c2 * LDX + rr] = da;
                pb[ii] = sum16(dn * sA[rr * LDX + c2]);
            }
        }
        if (isN && lm == 0) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sDb[(1 + x) * C + rb + 4 * lj + ii] = pb[ii];
        }
    } else {
        for (int e = tid - 384; e < 256; e += 128) {
            const int rr = e >> 4, c2 = 16 + (e & 15);
            sdP[rr * LDX + c2] = 0.f;
            sdPT[c2 * LDX + rr] = 0.f;
            sdA[rr * LDX + c2] = 0.f;
            sdAT[c2 * LDX + rr] = 0.f;
        }
        if (tid - 384 < 16) {     // rows that a block's dbeta part does not cover
            const int e = tid - 384;
            sDb[1 * C + 16 + e] = 0.f;
            sDb[2 * C + e] = 0.f;
            sDb[3 * C + e] = 0.f;
        }
    }
    __syncthreads();

    // ---- 4. token sums weighted by E, and the per-element results (channel cc)
    {
        const int c = cc;
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
            const int ta = 4 * lj + e, tb = 16 + 4 * lj + e;
            Kco[e] = kv(ta) * __expf((float)(g15 - gm(ta)));
            const float ro = __expf((float)(gm(tb) - g15));
            Kro[e] = kv(tb) * ro;
            Qro[e] = qv(tb) * ro;
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
                extra += kv(r) * dKh[rt][ii] * __expf((float)(gl - gm(r)));
            }
        extra = sum_rows4(extra) + dgm * __expf((float)gl);
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
                const float dq_ = dQp[rt][ii] * eG + dq2;
                const float dkrow = -sBeta[r] * dXS[rt][ii] * eG + dkr2;
                const float dkcol = dKh[rt][ii] * eGn + dkc2;
                const float kr = kv(r);
                float dG = qv(r) * dq_ + kr * dkrow - kr * dkcol;
                if (r == L - 1) dG += extra;
                if (r < L) {
                    dq[(int64_t)(c0 + r) * rowQ + hoff + c] = dq_;
                    dk[(int64_t)(c0 + r) * rowQ + hoff + c] = dkrow + dkcol;
                }
                sDG[r * LDF + c] = dG;    // sW's last reads were in part 3
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
        if (r < L) dbeta[(int64_t)(c0 + r) * H + h] = sDb[r] + sDb[C + r] + sDb[2 * C + r] + sDb[3 * C + r];
    }
}
}  // namespace kda

// Per (chunk, head) gradients of the chunk form (kda_bwd_chunk_kernel): S at
// every chunk start in snaps and the gradient at every chunk end in gchunk,
// both [chunks][H][BD][BD] as the chains store them (bf16: fp16 values with
// column scales [chunks][H][BD] in snap_scale / g_scale; fp32: fp32); every
// chunk's U, W (forward) and dX (state-gradient chain) [chunks][H][32][BD]
// fp32.  Writes dq, dk, dv, dg and dbeta.
extern "C" hipError_t kda_launch_bwd_chunk(int bf16, const void *q, const void *k, const float *g,
                                           const float *beta, const void *dout, const int32_t *cu,
                                           const int32_t *chunk_off, int64_t max_chunks, const void *snaps,
                                           const float *snap_scale, const void *gchunk, const float *g_scale,
                                           const float *uw_u, const float *uw_w, const float *dx_chunk, int32_t N,
                                           int32_t T_tot, int32_t H, float *dq, float *dk, float *dv, float *dg,
                                           float *dbeta, hipStream_t stream)
{
    using namespace kda;
    const int64_t grid = max_chunks * H;
    if (grid <= 0 || N <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (bf16 && (!snap_scale || !g_scale)) return hipErrorInvalidValue;
    if (bf16) {
        auto kern = kda_bwd_chunk_kernel<bf16_t>;
        static std::atomic<uint64_t> lds_set{0};
        if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(kern), (int)bc::Cfg<bf16_t>::bytes, lds_set))
            return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(bc::NT), bc::Cfg<bf16_t>::bytes, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k), g, beta,
                           static_cast<const bf16_t *>(dout), cu, chunk_off, snaps, snap_scale, gchunk, g_scale,
                           uw_u, uw_w, dx_chunk, N, T_tot, H, dq, dk, dv, dg, dbeta);
    } else {
        auto kern = kda_bwd_chunk_kernel<float>;
        static std::atomic<uint64_t> lds_set{0};
        if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(kern), (int)bc::Cfg<float>::bytes, lds_set))
            return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(bc::NT), bc::Cfg<float>::bytes, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k), g, beta,
                           static_cast<const float *>(dout), cu, chunk_off, snaps, snap_scale, gchunk, g_scale,
                           uw_u, uw_w, dx_chunk, N, T_tot, H, dq, dk, dv, dg, dbeta);
    }
    return hipGetLastError();
}
