// kda_decode.hip -- one KDA decode step (one new token per sequence and head).
//
// The step (page ailearn.mscapital.top/kimi-k3.html, card "KDA 单头递归"),
// with Sbar = Diag(exp(g)) S:
//     a = Sbar^T k,  b = Sbar^T q,  u = v - a,
//     S' = Sbar + beta k u^T,  o = S'^T q = b + beta (q.k) u,
// so one pass over the state yields both dk-reductions, and the state is read
// once and written once.  The kernel is bound by HBM traffic: 128 KiB of the
// 132.6 KB moved per (sequence, head) is the fp32 state.
//
// One workgroup (512 threads) per DEC_UNITS consecutive (sequence, head)
// pairs.  Thread t owns value columns 4*(t%32)..+3 and key rows (t/32) + 16*i,
// i = 0..7: every state row is read and written as 512 contiguous bytes
// (32 lanes x float4).  Partial reductions are combined across the 16 row
// groups through LDS.  The next pair's state is read while the current one
// is reduced and written back, so that a workgroup keeps reads in flight
// through its own write phase (the reduction over all key rows must finish
// before the first row can be written).
#include "kda_device.hpp"

namespace kda {

constexpr int D = 128;          // dk = dv
constexpr int DEC_THREADS = 512;
constexpr int ROWG = DEC_THREADS / 32;   // row groups
constexpr int RPT = D / ROWG;            // rows per thread
constexpr int DEC_UNITS = 2;             // (sequence, head) pairs per workgroup of the one-token step

// q, k, v, g, beta are not declared __restrict__: the compiler then keeps
// their loads in place, ahead of the state reads, instead of moving them next
// to their use, where waiting for them would also wait for the next pair's
// state (vector memory operations complete in order).
template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void kda_decode_kernel(
    const T *q, const T *k, const T *v, const float *g, const float *beta, float *state,
    T *__restrict__ out, int64_t units)
{
    __shared__ float sk[D], sq[D], sa[D];
    __shared__ f32x4 red_a[ROWG][D / 4], red_b[ROWG][D / 4];
    __shared__ float su[D];
    __shared__ float sqk;

    const int t = threadIdx.x;
    const int cg = t & 31, rg = t >> 5;
    const int64_t u0 = (int64_t)blockIdx.x * DEC_UNITS;
    const int nu = (int)min((int64_t)DEC_UNITS, units - u0);   // >= 1

    // the token vectors of every pair first, then the states in order
    T xk[DEC_UNITS], xq[DEC_UNITS], xv[DEC_UNITS];
    float xg[DEC_UNITS], xb[DEC_UNITS];
    {
        const int tt = t & (D - 1);
#pragma unroll
        for (int j = 0; j < DEC_UNITS; ++j) {
            const int64_t u = u0 + min(j, nu - 1);
            xk[j] = k[u * D + tt];
            xq[j] = q[u * D + tt];
            xg[j] = g[u * D + tt];
            xv[j] = v[u * D + tt];
            xb[j] = beta[u];
        }
    }
    f32x4 s[DEC_UNITS][RPT];
    // a pair past the end (last workgroup only) re-reads the last pair's
    // state, ahead of its update, and the values are dropped
    auto fetch = [&](int j) {
        const f32x4 *S4 = reinterpret_cast<const f32x4 *>(state + (u0 + min(j, nu - 1)) * (int64_t)D * D);
#pragma unroll
        for (int i = 0; i < RPT; ++i) s[j][i] = __builtin_nontemporal_load(&S4[(rg + ROWG * i) * (D / 4) + cg]);
        asm volatile("" ::: "memory");   // keep the reads here
    };
    fetch(0);
#pragma unroll
    for (int j = 0; j < DEC_UNITS; ++j) {
        if (j >= nu) break;
        if (j + 1 < DEC_UNITS) fetch(j + 1);
        const int64_t u = u0 + j;
        if (j > 0) __syncthreads();      // the previous pair is done with the LDS vectors
        if (t < D) {
            sk[t] = to_f(xk[j]);
            sq[t] = to_f(xq[j]);
            sa[t] = __expf(xg[j]);
        }
        __syncthreads();
        if (t < 64) {   // q.k by one wave
            float p = sk[t] * sq[t] + sk[t + 64] * sq[t + 64];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
            if (t == 0) sqk = p;
        }
        f32x4 pa = zero4(), pb = zero4();
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + ROWG * i;
            s[j][i] *= sa[r];
            pa += s[j][i] * sk[r];
            pb += s[j][i] * sq[r];
        }
        red_a[rg][cg] = pa;
        red_b[rg][cg] = pb;
        __syncthreads();
        const float bt = xb[j];
        if (t < D) {
            const int c4 = t >> 2, e = t & 3;
            float A = 0.f, B = 0.f;
#pragma unroll
            for (int r = 0; r < ROWG; ++r) {
                A += red_a[r][c4][e];
                B += red_b[r][c4][e];
            }
            const float uu = to_f(xv[j]) - A;
            su[t] = uu;
            out[u * D + t] = from_f<T>(B + bt * sqk * uu);
        }
        __syncthreads();
        const f32x4 uu = reinterpret_cast<const f32x4 *>(su)[cg];
        f32x4 *W4 = reinterpret_cast<f32x4 *>(state + u * (int64_t)D * D);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + ROWG * i;
            const f32x4 x = s[j][i] + (bt * sk[r]) * uu;
            __builtin_nontemporal_store(x, &W4[r * (D / 4) + cg]);
        }
    }
}


// Several consecutive tokens per (sequence, head) with the state kept in
// registers: it is read once and written at most once, whatever the number
// of tokens.  This serves speculative decoding (page section "目标模型太大，缓存
// 和草稿都必须理解 KDA": the projected inputs of draft tokens are cached, the
// accepted ones are replayed on chip, and a rejected draft is rolled back by
// not committing its state): verify a draft with state_out = NULL (outputs
// for every draft token, state untouched), then replay the accepted prefix
// with num_tokens = the accepted counts (state committed, out may be NULL).
// Per token the arithmetic is exactly that of kda_decode_kernel.
template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void kda_decode_tokens_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ num_tokens, const float *state_in, float *state_out,
    int32_t H, int32_t T_tot, T *__restrict__ out)
{
    __shared__ float sk[D], sq[D], sa[D];
    __shared__ f32x4 red_a[ROWG][D / 4], red_b[ROWG][D / 4];
    __shared__ float su[D];
    __shared__ float sqk;

    const int64_t u = blockIdx.x;                 // (sequence, head)
    const int n = (int)(u / H), h = (int)(u % H);
    const int t = threadIdx.x;
    const int cg = t & 31, rg = t >> 5;
    const int t0 = min(max(cu[n], 0), T_tot);
    int len = min(max(cu[n + 1], t0), T_tot) - t0;
    if (num_tokens) len = min(len, max(num_tokens[n], 0));

    f32x4 s[RPT];
    const f32x4 *S4 = reinterpret_cast<const f32x4 *>(state_in + u * (int64_t)D * D);
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(&S4[(rg + ROWG * i) * (D / 4) + cg]);

    for (int j = 0; j < len; ++j) {
        const int64_t row = (int64_t)(t0 + j) * H + h;    // this token of this head
        __syncthreads();                                 // previous token done with the LDS vectors
        if (t < D) {
            sk[t] = to_f(k[row * D + t]);
            sq[t] = to_f(q[row * D + t]);
            sa[t] = __expf(g[row * D + t]);
        }
        __syncthreads();
        if (t < 64) {   // q.k by one wave
            float p = sk[t] * sq[t] + sk[t + 64] * sq[t + 64];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
            if (t == 0) sqk = p;
        }
        f32x4 pa = zero4(), pb = zero4();
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + ROWG * i;
            s[i] *= sa[r];
            pa += s[i] * sk[r];
            pb += s[i] * sq[r];
        }
        red_a[rg][cg] = pa;
        red_b[rg][cg] = pb;
        __syncthreads();
        const float bt = beta[row];
        if (t < D) {
            const int c4 = t >> 2, e = t & 3;
            float A = 0.f, B = 0.f;
#pragma unroll
            for (int r = 0; r < ROWG; ++r) {
                A += red_a[r][c4][e];
                B += red_b[r][c4][e];
            }
            const float uu = to_f(v[row * D + t]) - A;
            su[t] = uu;
            if (out) out[row * D + t] = from_f<T>(B + bt * sqk * uu);
        }
        __syncthreads();
        const f32x4 uu = reinterpret_cast<const f32x4 *>(su)[cg];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + ROWG * i;
            s[i] = s[i] + (bt * sk[r]) * uu;
        }
    }

    if (state_out) {
        f32x4 *W4 = reinterpret_cast<f32x4 *>(state_out + u * (int64_t)D * D);
#pragma unroll
        for (int i = 0; i < RPT; ++i) __builtin_nontemporal_store(s[i], &W4[(rg + ROWG * i) * (D / 4) + cg]);
    }
}

}  // namespace kda

extern "C" hipError_t kda_launch_decode(int bf16, const void *q, const void *k, const void *v,
                                        const float *g, const float *beta, float *state,
                                        int32_t N, int32_t H, void *out, hipStream_t stream)
{
    using namespace kda;
    const int64_t units = (int64_t)N * H;
    if (units <= 0) return hipSuccess;
    if (units > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (bf16)
        hipLaunchKernelGGL(kda_decode_kernel<bf16_t>, dim3((unsigned)((units + DEC_UNITS - 1) / DEC_UNITS)), dim3(DEC_THREADS), 0, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k),
                           static_cast<const bf16_t *>(v), g, beta, state, static_cast<bf16_t *>(out), units);
    else
        hipLaunchKernelGGL(kda_decode_kernel<float>, dim3((unsigned)((units + DEC_UNITS - 1) / DEC_UNITS)), dim3(DEC_THREADS), 0, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(v), g, beta, state, static_cast<float *>(out), units);
    return hipGetLastError();
}

extern "C" hipError_t kda_launch_decode_tokens(int bf16, const void *q, const void *k, const void *v,
                                               const float *g, const float *beta, const int32_t *cu,
                                               const int32_t *num_tokens, const float *state_in,
                                               float *state_out, int32_t N, int32_t T_tot, int32_t H, void *out,
                                               hipStream_t stream)
{
    using namespace kda;
    const int64_t units = (int64_t)N * H;
    if (units <= 0) return hipSuccess;
    if (units > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (bf16)
        hipLaunchKernelGGL(kda_decode_tokens_kernel<bf16_t>, dim3((unsigned)units), dim3(DEC_THREADS), 0, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k),
                           static_cast<const bf16_t *>(v), g, beta, cu, num_tokens, state_in, state_out, H, T_tot,
                           static_cast<bf16_t *>(out));
    else
        hipLaunchKernelGGL(kda_decode_tokens_kernel<float>, dim3((unsigned)units), dim3(DEC_THREADS), 0, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(v), g, beta, cu, num_tokens, state_in, state_out, H, T_tot,
                           static_cast<float *>(out));
    return hipGetLastError();
}
