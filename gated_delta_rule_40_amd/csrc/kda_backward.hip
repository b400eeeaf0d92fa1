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
// from the state-gradient chain, S and G as those passes store them.  What is
// left here has no recurrence: one workgroup per (chunk, head).
// Precision: the Gram tile A and every 32-wide contraction run on fp32 (MFMA
// 16x16x4 and VALU).  The five 128-wide contractions (dQ+, dX S^T, dK^, dP,
// dN) run on the MFMA type of the forward: fp32 for fp32 inputs; fp16 for
// 16-bit inputs, with S and G read as the fp16 values and exact power-of-two
// column scales that the chains carry, and dO, W and dX held in fp16 with an
// exact power-of-two scale per row (the row maximum lands in [2^13, 2^14)); a
// product that needs another scale of a row, or a scale along the contraction
// index, rescales the fp16 values by an exact power of two, so every product
// is exact up to the fp16 rounding of its operands.
// Gamma: every decay factor is e^x of a difference of two cumulative gate
// entries.  For fp32 inputs Gamma is kept in fp64 and each difference rounded
// to fp32 only then, so a factor carries the rounding of its own exponent, not
// that of the (up to 160 in magnitude) cumulative sums; 16-bit inputs keep it
// in fp32, whose rounding (about 1e-5 of a factor) is far below their own.
// E is factored per 16-token block pair with a reference inside the pair --
// the middle token of a diagonal block, the block boundary for the
// off-diagonal one -- so every factor lies in [e^-80, e^40] for g in [-5, 0]:
// the Gram tile and the E-weighted token sums are then plain MFMA products of
// factored operands, and a factor applied after a product is at most e^40.
// Work split: four waves; in the key-channel parts wave w owns channels
// 32 w .. 32 w + 31 (two tiles); token rows are loaded by 16 lanes each (8
// columns per lane, two passes).  The 16-bit workgroup fits 80 KB of LDS, so
// two share a compute unit: one loads while the other computes.
namespace bc {
constexpr int C = 32, NW = 4, NT = 64 * NW, NCT = BD / (16 * NW);
constexpr int LDF = BD + 4;          // fp32 [C][BD] rows
constexpr int LDX = C + 4;           // fp32 [C][C] rows
constexpr int NDB = 4;               // partial dbeta slots: U.dX, and the dN (.) A part of 3 blocks
constexpr int NMX = 6;               // row scales from |dO|, |dO|/sS, |dX|, |dX|/sS, |W|, |W|/sG
enum { MX_DO = 0, MX_DOS = 1, MX_DX = 2, MX_DXS = 3, MX_W = 4, MX_WG = 5 };
template <typename T>
struct Cfg {
    static constexpr bool kIn16 = !std::is_same<T, float>::value;
    typedef typename std::conditional<kIn16, float, double>::type GT;   // cumulative gate
    typedef typename std::conditional<kIn16, f16_t, float>::type RT;    // dO, W, dX rows (row-scaled)
    static constexpr int LDI = BD + 16 / (int)sizeof(T);    // q, k rows (input type)
    static constexpr int LDG = BD + 16 / (int)sizeof(GT);   // Gamma rows
    static constexpr int LDR = BD + 16 / (int)sizeof(RT);   // dO, W, dX rows
    static constexpr uint32_t offK = 0;
    static constexpr uint32_t offQ = offK + sizeof(T) * C * LDI;
    static constexpr uint32_t offGm = offQ + sizeof(T) * C * LDI;
    static constexpr uint32_t offDO = offGm + sizeof(GT) * C * LDG;
    static constexpr uint32_t offW = offDO + sizeof(RT) * C * LDR;
    static constexpr uint32_t offDX = offW + sizeof(RT) * C * LDR;
    static constexpr uint32_t offA = offDX + sizeof(RT) * C * LDR;
    static constexpr uint32_t offdP = offA + sizeof(float) * C * LDX;     // first the Gram partials [3][256]
    static constexpr uint32_t offdA = offdP + sizeof(float) * C * LDX;
    static constexpr uint32_t offBeta = offdA + sizeof(float) * C * LDX;
    static constexpr uint32_t offDb = offBeta + sizeof(float) * C;        // [NDB][C] partial dbeta
    static constexpr uint32_t offIS = offDb + sizeof(float) * NDB * C;    // [BD] 1 / column scale of S
    static constexpr uint32_t offIG = offIS + sizeof(float) * BD;         // [BD] 1 / column scale of G
    static constexpr uint32_t offRS = offIG + sizeof(float) * BD;         // [NMX][C] row scales
    static constexpr uint32_t bytes = offRS + sizeof(float) * NMX * C;
    // dGamma (fp32 [C][LDF]) reuses the dO and W rows, dead after part 3
    static_assert(sizeof(float) * C * LDF <= offDX - offDO, "dGamma fits the dO and W rows");
    static_assert(3 * 256 * sizeof(float) <= sizeof(float) * C * LDX, "Gram partials fit dP");
    static_assert(bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
    static_assert(!kIn16 || bytes <= 80 * 1024, "two 16-bit workgroups per compute unit");
    static constexpr int WAVES_PER_EU = kIn16 ? 2 : 1;      // the register budget that allows it
};
typedef double f64x2 __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ f32x4 ld4(const T *p);
template <> __device__ __forceinline__ f32x4 ld4<float>(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
template <> __device__ __forceinline__ f32x4 ld4<bf16_t>(const bf16_t *p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{to_f(x[0]), to_f(x[1]), to_f(x[2]), to_f(x[3])};
}
template <> __device__ __forceinline__ f32x4 ld4<f16_t>(const f16_t *p) {
    const f16x4 x = *reinterpret_cast<const f16x4 *>(p);
    return f32x4{to_f(x[0]), to_f(x[1]), to_f(x[2]), to_f(x[3])};
}
// e^(a_e - b_e) for four consecutive Gamma entries, the differences in Gamma's type
__device__ __forceinline__ f32x4 exp_diff4(const double *a, const double *b) {
    const f64x2 a0 = *reinterpret_cast<const f64x2 *>(a), a1 = *reinterpret_cast<const f64x2 *>(a + 2);
    const f64x2 b0 = *reinterpret_cast<const f64x2 *>(b), b1 = *reinterpret_cast<const f64x2 *>(b + 2);
    return f32x4{__expf((float)(a0[0] - b0[0])), __expf((float)(a0[1] - b0[1])), __expf((float)(a1[0] - b1[0])),
                 __expf((float)(a1[1] - b1[1]))};
}
__device__ __forceinline__ f32x4 exp_diff4(const float *a, const float *b) {
    const f32x4 x = *reinterpret_cast<const f32x4 *>(a) - *reinterpret_cast<const f32x4 *>(b);
    return f32x4{__expf(x[0]), __expf(x[1]), __expf(x[2]), __expf(x[3])};
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
    // fragment of row `row` (elements of type OpT) as stored, no conversion
    __device__ static __forceinline__ typename M::frag raw(const OpT *row, int k0, int j) {
        typename M::frag f;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            typedef typename std::conditional<sizeof(OpT) == 2, f16x4, f32x4>::type V;
            const V x = *reinterpret_cast<const V *>(row + base(k0, j, gi));
#pragma unroll
            for (int e = 0; e < 4; ++e) f[4 * gi + e] = x[e];
        }
        return f;
    }
};
}  // namespace bc

// S (start state) and G (end gradient) of every chunk: [chunks][H][BD][BD] as
// the chains store them -- fp16 values with column scales [chunks][H][BD]
// (OpT = fp16) or fp32 (scales unused); U, W, dX: [chunks][H][C][BD] fp32.
template <typename T>
__global__ __launch_bounds__(bc::NT) __attribute__((amdgpu_waves_per_eu(bc::Cfg<T>::WAVES_PER_EU)))
void kda_bwd_chunk_kernel(
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
    constexpr bool kIn16 = Q::kIn16;
    typedef typename Q::GT GT;
    typedef typename Q::RT RT;
    typedef typename std::conditional<kIn16, f16_t, float>::type OpT;   // 128-wide contractions
    static_assert(std::is_same<OpT, RT>::value, "rows are stored in the operand type");
    typedef Mma<OpT> Mo;
    typedef Frag<OpT> F;
    constexpr int KB = Mo::KB, NG = F::NG;
    constexpr int LDI = Q::LDI, LDG = Q::LDG, LDR = Q::LDR;
    extern __shared__ __align__(16) unsigned char smem[];
    T *sK = reinterpret_cast<T *>(smem + Q::offK);
    T *sQ = reinterpret_cast<T *>(smem + Q::offQ);
    GT *sGm = reinterpret_cast<GT *>(smem + Q::offGm);
    RT *sDO = reinterpret_cast<RT *>(smem + Q::offDO);
    RT *sW = reinterpret_cast<RT *>(smem + Q::offW);
    RT *sDX = reinterpret_cast<RT *>(smem + Q::offDX);
    float *sA = reinterpret_cast<float *>(smem + Q::offA);
    float *sdP = reinterpret_cast<float *>(smem + Q::offdP);
    float *sdA = reinterpret_cast<float *>(smem + Q::offdA);
    float *sGp = sdP;
    float *sBeta = reinterpret_cast<float *>(smem + Q::offBeta);
    float *sDb = reinterpret_cast<float *>(smem + Q::offDb);
    float *sIS = reinterpret_cast<float *>(smem + Q::offIS);
    float *sIG = reinterpret_cast<float *>(smem + Q::offIG);
    float *sRS = reinterpret_cast<float *>(smem + Q::offRS);
    float *sDG = reinterpret_cast<float *>(smem + Q::offDO);

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
    // S and G rows of this lane's key channels for part 3 (tile ct: channel
    // 32 wave + 16 ct + lm), loaded first so that they arrive during parts 0-1
    typedef typename std::conditional<kIn16, f16x4, f32x4>::type V4;
    V4 spre[NCT][BD / KB][NG], gpre[NCT][BD / KB][NG];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int kb = 0; kb < BD / KB; ++kb)
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int64_t o = (int64_t)(32 * wave + 16 * ct + lm) * BD + F::base(kb * KB, lj, gi);
                spre[ct][kb][gi] = *reinterpret_cast<const V4 *>(Sg + o);
                gpre[ct][kb][gi] = *reinterpret_cast<const V4 *>(Gg + o);
            }

    // ---- 0. loads.  Thread (row r = tid / 16 + 16 pass, part m = tid % 16)
    //         takes columns 8 m .. 8 m + 7 of row r of q, k, dO, W, dX (and U,
    //         for the U.dX part of dbeta); a row's 16 parts are one DPP row,
    //         so its sums and maxima are taken across those lanes, and dO, W
    //         and dX are stored with their row scales.  Threads 0-127 also take
    //         channel tid of the gate for the cumulative sum.  Every global load
    //         is issued first, so that the part waits for memory once.
    {
        typedef typename std::conditional<kIn16, f32x4, f32x4[2]>::type Raw8;   // 8 input elements
        const int m = tid & 15, cb = 8 * m;
        Raw8 kraw[2], qraw[2], draw[2];
        f32x4 w[2][2], x[2][2], u[2][2], ss[2], sg[2];
        float br[2];
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const int r = (tid >> 4) + 16 * ps;
            const int64_t off = (int64_t)(c0 + min(r, L - 1)) * rowQ + hoff + cb;
            const int64_t cho = unit * C * BD + (int64_t)r * BD + cb;   // rows past the chunk: stored, not used
            if constexpr (kIn16) {
                kraw[ps] = *reinterpret_cast<const f32x4 *>(k + off);
                qraw[ps] = *reinterpret_cast<const f32x4 *>(q + off);
                draw[ps] = *reinterpret_cast<const f32x4 *>(dout + off);
            } else {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    kraw[ps][hf] = *reinterpret_cast<const f32x4 *>(k + off + 4 * hf);
                    qraw[ps][hf] = *reinterpret_cast<const f32x4 *>(q + off + 4 * hf);
                    draw[ps][hf] = *reinterpret_cast<const f32x4 *>(dout + off + 4 * hf);
                }
            }
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                w[ps][hf] = *reinterpret_cast<const f32x4 *>(uw_w + cho + 4 * hf);
                x[ps][hf] = *reinterpret_cast<const f32x4 *>(dx_chunk + cho + 4 * hf);
                u[ps][hf] = *reinterpret_cast<const f32x4 *>(uw_u + cho + 4 * hf);
            }
            br[ps] = beta[(int64_t)(c0 + min(r, L - 1)) * H + h];
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            ss[hf] = kIn16 ? *reinterpret_cast<const f32x4 *>(snap_scale + unit * BD + cb + 4 * hf) : f32x4{1.f, 1.f, 1.f, 1.f};
            sg[hf] = kIn16 ? *reinterpret_cast<const f32x4 *>(g_scale + unit * BD + cb + 4 * hf) : f32x4{1.f, 1.f, 1.f, 1.f};
        }
        float gv[C];
        if (tid < BD) {
#pragma unroll
            for (int i = 0; i < C; ++i) gv[i] = g[(int64_t)(c0 + min(i, L - 1)) * rowQ + hoff + tid];
        }
        asm volatile("" ::: "memory");                    // keeps the loads together
        f32x4 is[2], ig[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                is[hf][e] = pow2_inv(ss[hf][e]);
                ig[hf][e] = pow2_inv(sg[hf][e]);
            }
        if (tid < 16) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                *reinterpret_cast<f32x4 *>(sIS + cb + 4 * hf) = is[hf];
                *reinterpret_cast<f32x4 *>(sIG + cb + 4 * hf) = ig[hf];
            }
        }
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const int r = (tid >> 4) + 16 * ps;
            const bool ok = r < L;
            const int64_t off = (int64_t)(c0 + min(r, L - 1)) * rowQ + hoff + cb;
            if constexpr (kIn16) {
                *reinterpret_cast<f32x4 *>(sK + r * LDI + cb) = ok ? kraw[ps] : zero4();
                *reinterpret_cast<f32x4 *>(sQ + r * LDI + cb) = ok ? qraw[ps] : zero4();
            } else {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    *reinterpret_cast<f32x4 *>(sK + r * LDI + cb + 4 * hf) = ok ? kraw[ps][hf] : zero4();
                    *reinterpret_cast<f32x4 *>(sQ + r * LDI + cb + 4 * hf) = ok ? qraw[ps][hf] : zero4();
                }
            }
            f32x4 d[2];
            if constexpr (kIn16) {
                const bf16_t *db = reinterpret_cast<const bf16_t *>(&draw[ps]);
                d[0] = ld4(db);
                d[1] = ld4(db + 4);
            } else {
                d[0] = draw[ps][0];
                d[1] = draw[ps][1];
            }
            float ux = 0.f, mx[NMX] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                if (!ok) d[hf] = w[ps][hf] = x[ps][hf] = u[ps][hf] = zero4();
                ux += dot4(u[ps][hf], x[ps][hf]);
                mx[MX_DO] = fmaxf(mx[MX_DO], max4(abs4(d[hf])));
                mx[MX_DOS] = fmaxf(mx[MX_DOS], max4(abs4(d[hf]) * is[hf]));
                mx[MX_DX] = fmaxf(mx[MX_DX], max4(abs4(x[ps][hf])));
                mx[MX_DXS] = fmaxf(mx[MX_DXS], max4(abs4(x[ps][hf]) * is[hf]));
                mx[MX_W] = fmaxf(mx[MX_W], max4(abs4(w[ps][hf])));
                mx[MX_WG] = fmaxf(mx[MX_WG], max4(abs4(w[ps][hf]) * ig[hf]));
            }
            if (ok) {                                     // dv = Diag(b) dX
                *reinterpret_cast<f32x4 *>(dv + off) = x[ps][0] * br[ps];
                *reinterpret_cast<f32x4 *>(dv + off + 4) = x[ps][1] * br[ps];
            }
            ux = sum16(ux);
            float rs[NMX];
#pragma unroll
            for (int a = 0; a < NMX; ++a) rs[a] = kIn16 ? pow2_scale(rowmax16(mx[a])) : 1.f;
            // dO, W, dX rows in the operand type with their row scales
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sDO[r * LDR + cb + 4 * hf + e] = from_f<RT>(d[hf][e] * rs[MX_DO]);
                    sW[r * LDR + cb + 4 * hf + e] = from_f<RT>(w[ps][hf][e] * rs[MX_W]);
                    sDX[r * LDR + cb + 4 * hf + e] = from_f<RT>(x[ps][hf][e] * rs[MX_DX]);
                }
            if (m == 0) {
                sDb[r] = ux;
                sBeta[r] = ok ? br[ps] : 0.f;
#pragma unroll
                for (int a = 0; a < NMX; ++a) sRS[a * C + r] = rs[a];
            }
        }
        if (tid < BD) {
            GT sum = 0;
#pragma unroll
            for (int i = 0; i < C; ++i) {
                if (i < L) sum += (GT)gv[i];
                sGm[i * LDG + tid] = sum;
            }
        }
    }
    __syncthreads();

    // ---- 1. Gram tile A (strictly lower): block x = wave for waves 0-2, x = 0,
    //         1 diagonal (reference: the block's middle token), x = 2 the
    //         off-diagonal one (reference: token 15); wave 3 zeroes the upper block
    if (wave < 3) {
        const int x = wave;
        const int rb = x == 0 ? 0 : 16, ib = x == 1 ? 16 : 0, ref = x == 0 ? 7 : (x == 1 ? 23 : 15);
        const int r = rb + lm, i = ib + lm;
        f32x4 acc = zero4();
#pragma unroll 4
        for (int kb = 0; kb < BD / 16; ++kb) {
            const int c = 16 * kb + 4 * lj;
            const f32x4 rf = exp_diff4(sGm + r * LDG + c, sGm + ref * LDG + c);
            const f32x4 cf = exp_diff4(sGm + ref * LDG + c, sGm + i * LDG + c);
            acc = Mf::mma(ld4(sK + r * LDI + c) * rf, ld4(sK + i * LDI + c) * cf, acc);
        }
        const bool diag = x < 2;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int rr = rb + 4 * lj + ii, cc = ib + lm;
            sA[rr * LDX + cc] = (!diag || cc < rr) ? acc[ii] : 0.f;   // a select: entries above may be inf
        }
    } else {
        for (int e = lane; e < 256; e += 64) sA[(e >> 4) * LDX + 16 + (e & 15)] = 0.f;
    }
    __syncthreads();

    // ---- 3. contractions over the value columns, on the MFMA type of the
    //         forward: key channels 32 wave + 16 ct + lm of this lane; S and G
    //         rows as prefetched (the fragment's indices along the row)
    f32x4 dQp[NCT][2], dXS[NCT][2], dKh[NCT][2];
    float dgm[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        dgm[ct] = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) dQp[ct][rt] = dXS[ct][rt] = dKh[ct][rt] = zero4();
    }
#pragma unroll
    for (int kb = 0; kb < BD / KB; ++kb) {
        typename Mo::frag st[NCT], gt[NCT];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int j = F::base(kb * KB, lj, gi);
            const f32x4 isv = ld4(sIS + j), igv = ld4(sIG + j);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    st[ct][4 * gi + e] = spre[ct][kb][gi][e];
                    gt[ct][4 * gi + e] = gpre[ct][kb][gi][e];
                    dgm[ct] += (float)spre[ct][kb][gi][e] * isv[e] * ((float)gpre[ct][kb][gi][e] * igv[e]);
                }
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int r = 16 * rt + lm;
            // rows stored with the scales MX_DO, MX_DX, MX_W; here they enter
            // with MX_DOS, MX_DXS, MX_WG and a column factor 1/sS or 1/sG
            const float fdo = sRS[MX_DOS * C + r] * pow2_inv(sRS[MX_DO * C + r]);
            const float fdx = sRS[MX_DXS * C + r] * pow2_inv(sRS[MX_DX * C + r]);
            const float fw = sRS[MX_WG * C + r] * pow2_inv(sRS[MX_W * C + r]);
            f32x4 ado[NG], adx[NG], aw[NG];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int j = F::base(kb * KB, lj, gi);
                const f32x4 isv = ld4(sIS + j), igv = ld4(sIG + j);
                ado[gi] = ld4(sDO + r * LDR + j) * isv;
                adx[gi] = ld4(sDX + r * LDR + j) * isv;
                aw[gi] = ld4(sW + r * LDR + j) * igv;
            }
            const typename Mo::frag fo = F::make(ado, fdo), fx = F::make(adx, fdx), fwf = F::make(aw, fw);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                dQp[ct][rt] = Mo::mma(fo, st[ct], dQp[ct][rt]);
                dXS[ct][rt] = Mo::mma(fx, st[ct], dXS[ct][rt]);
                dKh[ct][rt] = Mo::mma(fwf, gt[ct], dKh[ct][rt]);
            }
        }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        dgm[ct] = sum_rows4(dgm[ct]);                     // (G (.) S) 1 of the channel
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {                 // undo the row scales
                const int r = 16 * rt + 4 * lj + i;
                dQp[ct][rt][i] *= pow2_inv(sRS[MX_DOS * C + r]);
                dXS[ct][rt][i] *= pow2_inv(sRS[MX_DXS * C + r]);
                dKh[ct][rt][i] *= pow2_inv(sRS[MX_WG * C + r]);
            }
    }
    // dP and dN by block x (jobs 0-2: dP, 3-5: dN; wave w takes jobs w and w + 4),
    // A = dO or dX rows and B = W rows as stored; wave 3 also zeroes the upper blocks
#pragma unroll 1
    for (int job = wave; job < 6; job += NW) {
        const int x = job % 3;
        const bool isN = job >= 3, diag = x < 2;
        const int rb = x == 0 ? 0 : 16, ib = x == 1 ? 16 : 0;
        const RT *rowA = (isN ? sDX : sDO) + (rb + lm) * LDR;
        const RT *rowB = sW + (ib + lm) * LDR;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < BD / KB; ++kb) acc = Mo::mma(F::raw(rowA, kb * KB, lj), F::raw(rowB, kb * KB, lj), acc);
        const float iw = pow2_inv(sRS[MX_W * C + ib + lm]);
        float pb[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int rr = rb + 4 * lj + ii, c2 = ib + lm;
            const float val = acc[ii] * pow2_inv(sRS[(isN ? MX_DX : MX_DO) * C + rr]) * iw;
            if (!isN) {
                sdP[rr * LDX + c2] = (!diag || c2 <= rr) ? val : 0.f;
                pb[ii] = 0.f;
            } else {
                const float dn = (!diag || c2 < rr) ? -val : 0.f;
                sdA[rr * LDX + c2] = sBeta[rr] * dn;
                pb[ii] = sum16(dn * sA[rr * LDX + c2]);
            }
        }
        if (isN && lm == 0) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sDb[(1 + x) * C + rb + 4 * lj + ii] = pb[ii];
        }
    }
    if (wave == NW - 1) {
        for (int e = lane; e < 256; e += 64) {
            const int rr = e >> 4, c2 = 16 + (e & 15);
            sdP[rr * LDX + c2] = 0.f;
            sdA[rr * LDX + c2] = 0.f;
        }
        if (lane < 16) {          // rows that a block's dbeta part does not cover
            sDb[1 * C + 16 + lane] = 0.f;
            sDb[2 * C + lane] = 0.f;
            sDb[3 * C + lane] = 0.f;
        }
    }
    __syncthreads();

    // ---- 4. token sums weighted by E, and the per-element results
    //         (dGamma to LDS over the dO and W rows, dead since part 3)
#pragma unroll 1
    for (int ct = 0; ct < NCT; ++ct) {
        const int c = 32 * wave + 16 * ct + lm;
        // this tile's products by selects over the tiles (compile-time indices:
        // indexed by the loop's ct they would go through scratch memory, whose
        // loads wait for the previous tile's dq / dk stores)
        f32x4 cQp[2], cXS[2], cKh[2];
        float cgm = dgm[0];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            cQp[rt] = dQp[0][rt];
            cXS[rt] = dXS[0][rt];
            cKh[rt] = dKh[0][rt];
        }
#pragma unroll
        for (int t = 1; t < NCT; ++t)
            if (ct == t) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    cQp[rt] = dQp[t][rt];
                    cXS[rt] = dXS[t][rt];
                    cKh[rt] = dKh[t][rt];
                }
                cgm = dgm[t];
            }
        auto gm = [&](int t) { return sGm[t * LDG + c]; };
        auto kv = [&](int t) { return to_f(sK[t * LDI + c]); };
        auto qv = [&](int t) { return to_f(sQ[t * LDI + c]); };
        // transposed A operands: lane row m reads column m of dP / dA
        auto colA = [&](const float *M, int col, int r0) {
            return f32x4{M[(r0 + 0) * LDX + col], M[(r0 + 1) * LDX + col], M[(r0 + 2) * LDX + col],
                         M[(r0 + 3) * LDX + col]};
        };
        // B operands over tokens: lane group lj takes tokens tb + 4 lj + e
        f32x4 Kcd[2], Krd[2], Qrd[2], Kco, Kro, Qro;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const GT gmid = gm(16 * a + 7);
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
        const GT g15 = gm(15);
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
            kc2d[a] = Mf::mma(colA(sdA, 16 * a + lm, 16 * a + 4 * lj), Krd[a],
                              Mf::mma(colA(sdP, 16 * a + lm, 16 * a + 4 * lj), Qrd[a], zero4()));
        }
        const f32x4 q2o = Mf::mma(ld4(sdP + (16 + lm) * LDX + 4 * lj), Kco, zero4());
        const f32x4 kr2o = Mf::mma(ld4(sdA + (16 + lm) * LDX + 4 * lj), Kco, zero4());
        const f32x4 kc2o = Mf::mma(colA(sdA, lm, 16 + 4 * lj), Kro, Mf::mma(colA(sdP, lm, 16 + 4 * lj), Qro, zero4()));
        // the last token's extra terms: sum_r k dK^ e^(Gamma_L - Gamma) and (G (.) S) 1 e^Gamma_L
        const GT gl = gm(L - 1);
        float extra = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int r = 16 * rt + 4 * lj + ii;
                extra += kv(r) * cKh[rt][ii] * __expf((float)(gl - gm(r)));
            }
        extra = sum_rows4(extra) + cgm * __expf((float)gl);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int r = 16 * rt + 4 * lj + ii;
                const GT gr = gm(r), gmid = gm(16 * rt + 7);
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
                const float dq_ = cQp[rt][ii] * eG + dq2;
                const float dkrow = -sBeta[r] * cXS[rt][ii] * eG + dkr2;
                const float dkcol = cKh[rt][ii] * eGn + dkc2;
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
        // every row read first (one batch of LDS reads, not one round trip
        // per row), then summed from the last valid row down, as before
        float dgr[C];
#pragma unroll
        for (int r = 0; r < C; ++r) dgr[r] = sDG[r * LDF + tid];
        float acc = 0.f;
#pragma unroll
        for (int r = C - 1; r >= 0; --r)
            if (r < L) {
                acc += dgr[r];
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
