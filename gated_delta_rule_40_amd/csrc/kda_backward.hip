// kda_backward.hip -- gradients of the KDA recurrence (training).
//
// The recurrence (page ailearn.mscapital.top/kimi-k3.html, card "KDA 单头递归"),
// token form with Sp = S_{t-1}, alpha = exp(g):
//     Sbar = Diag(alpha) Sp,  u = v - Sbar^T k,  S = Sbar + beta k u^T,  o = S^T q.
// Its reverse, for dS = dL/dS_t (from later tokens, or d(final_state)):
//     dS  += q do^T;            dq = S do
//     x    = dS^T k;            du = dv = beta x;       dbeta = x . u
//     dk   = beta dS u - Sbar du
//     dSbar = dS - k du^T;      dg = alpha (.) rowsum(dSbar (.) Sp)
//     dS_{t-1} = Diag(alpha) dSbar
// and d(initial_state) is dS after the first token.
//
// Work decomposition.  The state and its gradient evolve column by column:
// column c of S and dS needs only column c of v, do and du.  Only dq, dk, dg
// and dbeta sum over columns.  So one workgroup owns a (sequence, head) and a
// block of BV = 32 value columns, with S and dS in registers; its row sums go
// to per-block partial buffers that a second kernel adds in a fixed order
// (deterministic).  The forward states are needed in reverse order: the
// state at every 32-token chunk start comes from the forward prefill kernel
// (snapshot mode), and inside a chunk the workgroup recomputes the 32 token
// states into its own scratch area, then walks them backwards.
#include "kda_device.hpp"

namespace kda {

constexpr int BD = 128;              // dk = dv
constexpr int BWD_THREADS = 256;
constexpr int BWD_C = 32;            // tokens per checkpoint interval (the forward chunk)
constexpr int BWD_BV = 32;           // value columns per workgroup
constexpr int BWD_CPR = BWD_BV / 4;  // threads per row group (4 columns each)
constexpr int BWD_RG = BWD_THREADS / BWD_CPR;   // row groups
constexpr int BWD_RPT = BD / BWD_RG;            // rows per thread
constexpr int BWD_NBLK = BD / BWD_BV;
static_assert(BWD_CPR == 8, "row sums use sum8");

__device__ __forceinline__ float dot4(const f32x4 &a, const f32x4 &b) {
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// part_vec: [NBLK][3][T_tot * H][BD] partial row sums (dq, dk, dg);
// part_beta: [NBLK][T_tot * H]; scratch: [N * H * NBLK][BWD_C][BD][BWD_BV];
// snaps: [chunks][H][BD][BD], the state at the start of global chunk
// chunk_off[n] + c for c >= 1 (c = 0 is the initial state).
template <typename T>
__global__ __launch_bounds__(BWD_THREADS) void kda_backward_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *initial_state,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, const float *__restrict__ snaps,
    const T *__restrict__ dout, const float *dfinal, int32_t H, int32_t T_tot,
    float *__restrict__ scratch, float *__restrict__ part_vec, float *__restrict__ part_beta,
    float *__restrict__ dv_out, float *dinit)
{
    __shared__ float sq[BD], sk[BD], sa[BD];
    __shared__ float sv[BWD_BV], sdo[BWD_BV], su[BWD_BV], sx[BWD_BV];
    __shared__ f32x4 red_a[BWD_RG][BWD_CPR], red_x[BWD_RG][BWD_CPR];

    const int blk = blockIdx.x % BWD_NBLK;
    const int64_t unit = blockIdx.x / BWD_NBLK;
    const int n = (int)(unit / H), h = (int)(unit % H);
    const int t = threadIdx.x;
    const int cg = t % BWD_CPR, rg = t / BWD_CPR;
    const int dv0 = blk * BWD_BV, c4 = dv0 + 4 * cg;
    const int t0 = min(max(cu[n], 0), T_tot);
    const int t1 = min(max(cu[n + 1], t0), T_tot);
    const int nch = (t1 - t0 + BWD_C - 1) / BWD_C;
    const int64_t sbase = unit * BD * BD;              // this (sequence, head) in [N, H, BD, BD]
    const int64_t rows_all = (int64_t)T_tot * H;
    float *scr = scratch + ((int64_t)unit * BWD_NBLK + blk) * BWD_C * BD * BWD_BV;

    f32x4 S[BWD_RPT], dS[BWD_RPT], Sp[BWD_RPT];
#pragma unroll
    for (int i = 0; i < BWD_RPT; ++i) {
        const int r = rg + BWD_RG * i;
        dS[i] = dfinal ? *reinterpret_cast<const f32x4 *>(dfinal + sbase + (int64_t)r * BD + c4) : zero4();
    }

    for (int c = nch - 1; c >= 0; --c) {
        const int c0 = t0 + c * BWD_C, Lc = min(BWD_C, t1 - c0);
        const float *src = c ? snaps + ((int64_t)(chunk_off[n] + c) * H + h) * BD * BD
                             : (initial_state ? initial_state + sbase : nullptr);
#pragma unroll
        for (int i = 0; i < BWD_RPT; ++i) {
            const int r = rg + BWD_RG * i;
            S[i] = src ? *reinterpret_cast<const f32x4 *>(src + (int64_t)r * BD + c4) : zero4();
        }

        // ---- forward inside the chunk: scr[j] = state before token c0 + j
        for (int j = 0; j < Lc; ++j) {
            const int64_t row = (int64_t)(c0 + j) * H + h;
#pragma unroll
            for (int i = 0; i < BWD_RPT; ++i)
                *reinterpret_cast<f32x4 *>(scr + ((int64_t)j * BD + rg + BWD_RG * i) * BWD_BV + 4 * cg) = S[i];
            __syncthreads();                                   // token vectors free
            if (t < BD) {
                sk[t] = to_f(k[row * BD + t]);
                sa[t] = __expf(g[row * BD + t]);
            }
            if (t < BWD_BV) sv[t] = to_f(v[row * BD + dv0 + t]);
            __syncthreads();
            const float bt = beta[row];
            f32x4 pa = zero4();
#pragma unroll
            for (int i = 0; i < BWD_RPT; ++i) {
                const int r = rg + BWD_RG * i;
                S[i] *= sa[r];
                pa += S[i] * sk[r];
            }
            red_a[rg][cg] = pa;
            __syncthreads();
            if (t < BWD_BV) {
                float A = 0.f;
                for (int r = 0; r < BWD_RG; ++r) A += red_a[r][t >> 2][t & 3];
                su[t] = sv[t] - A;
            }
            __syncthreads();
            const f32x4 u4 = *reinterpret_cast<const f32x4 *>(su + 4 * cg);
#pragma unroll
            for (int i = 0; i < BWD_RPT; ++i) S[i] += (bt * sk[rg + BWD_RG * i]) * u4;
        }

        // ---- reverse over the chunk's tokens
        for (int j = Lc - 1; j >= 0; --j) {
            const int64_t row = (int64_t)(c0 + j) * H + h;
#pragma unroll
            for (int i = 0; i < BWD_RPT; ++i)
                Sp[i] = *reinterpret_cast<const f32x4 *>(scr + ((int64_t)j * BD + rg + BWD_RG * i) * BWD_BV + 4 * cg);
            __syncthreads();
            if (t < BD) {
                sq[t] = to_f(q[row * BD + t]);
                sk[t] = to_f(k[row * BD + t]);
                sa[t] = __expf(g[row * BD + t]);
            }
            if (t < BWD_BV) {
                sv[t] = to_f(v[row * BD + dv0 + t]);
                sdo[t] = to_f(dout[row * BD + dv0 + t]);
            }
            __syncthreads();
            const float bt = beta[row];
            const f32x4 do4 = *reinterpret_cast<const f32x4 *>(sdo + 4 * cg);
            f32x4 pa = zero4(), px = zero4();
#pragma unroll
            for (int i = 0; i < BWD_RPT; ++i) {
                const int r = rg + BWD_RG * i;
                pa += (Sp[i] * sa[r]) * sk[r];                 // Sbar^T k
                dS[i] += sq[r] * do4;                          // o = S^T q
                px += dS[i] * sk[r];                           // dS^T k
            }
            red_a[rg][cg] = pa;
            red_x[rg][cg] = px;
            __syncthreads();
            if (t < BWD_BV) {
                float A = 0.f, X = 0.f;
                for (int r = 0; r < BWD_RG; ++r) {
                    A += red_a[r][t >> 2][t & 3];
                    X += red_x[r][t >> 2][t & 3];
                }
                su[t] = sv[t] - A;
                sx[t] = X;
                dv_out[row * BD + dv0 + t] = bt * X;
            }
            __syncthreads();
            const f32x4 u4 = *reinterpret_cast<const f32x4 *>(su + 4 * cg);
            const f32x4 du4 = *reinterpret_cast<const f32x4 *>(sx + 4 * cg) * bt;
            float pq[BWD_RPT], pk[BWD_RPT], pg[BWD_RPT];
#pragma unroll
            for (int i = 0; i < BWD_RPT; ++i) {
                const int r = rg + BWD_RG * i;
                const float a = sa[r], kr = sk[r];
                const f32x4 sb = Sp[i] * a;
                const f32x4 sn = sb + (bt * kr) * u4;
                pq[i] = dot4(sn, do4);
                pk[i] = bt * dot4(dS[i], u4) - dot4(sb, du4);
                const f32x4 dsb = dS[i] - kr * du4;
                pg[i] = a * dot4(dsb, Sp[i]);
                dS[i] = dsb * a;
            }
#pragma unroll
            for (int i = 0; i < BWD_RPT; ++i) {
                pq[i] = sum8(pq[i]);
                pk[i] = sum8(pk[i]);
                pg[i] = sum8(pg[i]);
            }
            if (cg == 0) {
                float *pv = part_vec + (int64_t)blk * 3 * rows_all * BD + row * BD;
#pragma unroll
                for (int i = 0; i < BWD_RPT; ++i) {
                    const int r = rg + BWD_RG * i;
                    pv[r] = pq[i];
                    pv[rows_all * BD + r] = pk[i];
                    pv[2 * rows_all * BD + r] = pg[i];
                }
            }
            if (t < 64) {   // dbeta over this block's columns (wave 0)
                const float p = wavesum(t < BWD_BV ? sx[t] * su[t] : 0.f);
                if (t == 0) part_beta[(int64_t)blk * rows_all + row] = p;
            }
        }
    }

    if (dinit) {
#pragma unroll
        for (int i = 0; i < BWD_RPT; ++i) {
            const int r = rg + BWD_RG * i;
            *reinterpret_cast<f32x4 *>(dinit + sbase + (int64_t)r * BD + c4) = dS[i];
        }
    }
}

// Sum of the per-block partials in block order: dq, dk, dg [rows][BD], dbeta [rows].
// Rows of tokens outside every sequence are written as zeros in the partials'
// place only if a workgroup wrote them; the caller's rows are selected by row_ok.
__global__ __launch_bounds__(256) void kda_backward_reduce_kernel(
    const float *__restrict__ part_vec, const float *__restrict__ part_beta, const int32_t *__restrict__ cu,
    int32_t N, int32_t H, int64_t rows_all, float *__restrict__ dq, float *__restrict__ dk,
    float *__restrict__ dg, float *__restrict__ dbeta)
{
    const int64_t nvec = rows_all * (BD / 4);
    const int32_t t_lo = min(max(cu[0], 0), (int32_t)(rows_all / H));
    const int32_t t_hi = min(max(cu[N], t_lo), (int32_t)(rows_all / H));
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < nvec; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = e / (BD / 4);
        const int32_t tok = (int32_t)(row / H);
        if (tok < t_lo || tok >= t_hi) continue;        // tokens outside the packed sequences
        f32x4 a = zero4(), b = zero4(), c = zero4();
#pragma unroll
        for (int blk = 0; blk < BWD_NBLK; ++blk) {
            const f32x4 *pv = reinterpret_cast<const f32x4 *>(part_vec + (int64_t)blk * 3 * rows_all * BD);
            a += pv[e];
            b += pv[nvec + e];
            c += pv[2 * nvec + e];
        }
        reinterpret_cast<f32x4 *>(dq)[e] = a;
        reinterpret_cast<f32x4 *>(dk)[e] = b;
        reinterpret_cast<f32x4 *>(dg)[e] = c;
        if ((e % (BD / 4)) == 0) {
            float s = 0.f;
#pragma unroll
            for (int blk = 0; blk < BWD_NBLK; ++blk) s += part_beta[(int64_t)blk * rows_all + row];
            dbeta[row] = s;
        }
    }
}

}  // namespace kda

extern "C" size_t kda_backward_scratch_floats_per_unit() { return (size_t)kda::BWD_NBLK * kda::BWD_C * kda::BD * kda::BWD_BV; }
extern "C" int32_t kda_backward_num_blocks() { return kda::BWD_NBLK; }

extern "C" hipError_t kda_launch_backward(int bf16, const void *q, const void *k, const void *v, const float *g,
                                          const float *beta, const float *init, const int32_t *cu,
                                          const int32_t *chunk_off, const float *snaps, const void *dout,
                                          const float *dfinal, int32_t N, int32_t T_tot, int32_t H, float *scratch,
                                          float *part_vec, float *part_beta, float *dq, float *dk, float *dv,
                                          float *dg, float *dbeta, float *dinit, hipStream_t stream)
{
    using namespace kda;
    const int64_t grid = (int64_t)N * H * BWD_NBLK;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (bf16)
        hipLaunchKernelGGL(kda_backward_kernel<bf16_t>, dim3((unsigned)grid), dim3(BWD_THREADS), 0, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k),
                           static_cast<const bf16_t *>(v), g, beta, init, cu, chunk_off, snaps,
                           static_cast<const bf16_t *>(dout), dfinal, H, T_tot, scratch, part_vec, part_beta, dv,
                           dinit);
    else
        hipLaunchKernelGGL(kda_backward_kernel<float>, dim3((unsigned)grid), dim3(BWD_THREADS), 0, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(v), g, beta, init, cu, chunk_off, snaps,
                           static_cast<const float *>(dout), dfinal, H, T_tot, scratch, part_vec, part_beta, dv,
                           dinit);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows_all = (int64_t)T_tot * H;
    const int64_t nvec = rows_all * (BD / 4);
    if (nvec == 0) return hipSuccess;
    const int64_t blocks = min((nvec + 255) / 256, (int64_t)65536);
    hipLaunchKernelGGL(kda_backward_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part_vec, part_beta,
                       cu, N, H, rows_all, dq, dk, dg, dbeta);
    return hipGetLastError();
}
