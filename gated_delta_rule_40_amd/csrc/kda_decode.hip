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
// Per token the arithmetic is exactly that of kda_decode_kernel, in the same
// thread layout.  As there, a workgroup takes DEC_UNITS consecutive (sequence,
// head) pairs and reads the next pair's state while the current one is
// processed and written.  The token vectors of a pair's first TOK_STAGED
// tokens are read up front, before that prefetch, so that no later wait sits
// behind it (vector memory operations complete in order); further tokens are
// read when they are reached.  Thread t stages element t % 128 of vector
// t / 128 (k, q, v, g) of a token as the 32-bit word holding it: one load per
// thread and token, picked by pointer, with no branch around a load (a load
// under a branch makes the compiler wait for it at once).  Requires T_tot > 0.
constexpr int TOK_STAGED = 4;
template <typename T>
__global__ __launch_bounds__(DEC_THREADS) __attribute__((amdgpu_waves_per_eu(4)))   // two workgroups per CU
void kda_decode_tokens_kernel(
    const T *q, const T *k, const T *v, const float *g, const float *beta, const int32_t *cu,
    const int32_t *num_tokens, const float *state_in, float *state_out,
    int32_t H, int32_t T_tot, int64_t units, T *__restrict__ out)
{
    __shared__ float svec[4][D];            // k, q, v, exp(g) of the current token
    __shared__ f32x4 red_a[ROWG][D / 4], red_b[ROWG][D / 4];
    __shared__ float su[D];
    __shared__ float sqk;
    float *const sk = svec[0], *const sq = svec[1], *const sv = svec[2], *const sa = svec[3];

    const int t = threadIdx.x;
    const int cg = t & 31, rg = t >> 5;
    const int vi = t / D, e = t % D;        // staged vector (0 k, 1 q, 2 v, 3 g) and element
    const int64_t u0 = (int64_t)blockIdx.x * DEC_UNITS;
    const int nu = (int)min((int64_t)DEC_UNITS, units - u0);   // >= 1

    // sequence bounds of every pair first (no branch: without num_tokens the
    // count is read from cu and not used)
    int c0[DEC_UNITS], c1[DEC_UNITS], cn[DEC_UNITS], hh[DEC_UNITS];
#pragma unroll
    for (int j = 0; j < DEC_UNITS; ++j) {
        const int64_t u = u0 + min(j, nu - 1);
        const int n = (int)(u / H);
        hh[j] = (int)(u % H);
        c0[j] = cu[n];
        c1[j] = cu[n + 1];
        cn[j] = (num_tokens ? num_tokens : cu)[n];
    }
    f32x4 s[DEC_UNITS][RPT];
    // a pair past the end (last workgroup only) re-reads the last pair, whose
    // values are dropped; its state is read ahead of any update of it
    auto fetch_state = [&](int j) {
        const f32x4 *S4 = reinterpret_cast<const f32x4 *>(state_in + (u0 + min(j, nu - 1)) * (int64_t)D * D);
#pragma unroll
        for (int i = 0; i < RPT; ++i) s[j][i] = __builtin_nontemporal_load(&S4[(rg + ROWG * i) * (D / 4) + cg]);
        asm volatile("" ::: "memory");
    };
    fetch_state(0);
    int t0[DEC_UNITS], len[DEC_UNITS];
#pragma unroll
    for (int j = 0; j < DEC_UNITS; ++j) {
        t0[j] = min(max(c0[j], 0), T_tot);
        len[j] = min(max(c1[j], t0[j]), T_tot) - t0[j];
        if (num_tokens) len[j] = min(len[j], max(cn[j], 0));
    }

    // this thread's staged vector as bytes, and its element size
    const unsigned char *vbase = reinterpret_cast<const unsigned char *>(
        vi == 0 ? (const void *)k : vi == 1 ? (const void *)q : vi == 2 ? (const void *)v : (const void *)g);
    const int esz = vi == 3 ? 4 : (int)sizeof(T);
    auto load_word = [&](int64_t row) {
        const int64_t off = (row * D + e) * esz;
        return *reinterpret_cast<const uint32_t *>(vbase + (off & ~(int64_t)3));
    };
    // value of the staged element from its word
    auto word_value = [&](uint32_t w) {
        if (vi == 3 || sizeof(T) == 4) return __uint_as_float(w);
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));   // bf16 -> fp32 (exact)
    };
    auto token_row = [&](int j, int jj) {   // clamped into [0, T_tot): a token past the count is dropped
        const int tok = min(t0[j] + min(jj, max(len[j] - 1, 0)), T_tot - 1);
        return (int64_t)tok * H + hh[j];
    };
    uint32_t xw[DEC_UNITS][TOK_STAGED];
    float xb[DEC_UNITS][TOK_STAGED];
#pragma unroll
    for (int j = 0; j < DEC_UNITS; ++j)
#pragma unroll
        for (int jj = 0; jj < TOK_STAGED; ++jj) {
            const int64_t row = token_row(j, jj);
            xw[j][jj] = load_word(row);
            xb[j][jj] = beta[row];
        }
    asm volatile("" ::: "memory");

    // one token: the decode step on the state registers of pair j
    auto step = [&](int j, int jj, uint32_t w, float bt) {
        __syncthreads();                                 // previous token done with the LDS vectors
        const float x = word_value(w);
        svec[vi][e] = vi == 3 ? __expf(x) : x;
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
        if (t < D) {
            const int c4 = t >> 2, e4 = t & 3;
            float A = 0.f, B = 0.f;
#pragma unroll
            for (int r = 0; r < ROWG; ++r) {
                A += red_a[r][c4][e4];
                B += red_b[r][c4][e4];
            }
            const float uu = sv[t] - A;
            su[t] = uu;
            if (out) out[((int64_t)(t0[j] + jj) * H + hh[j]) * D + t] = from_f<T>(B + bt * sqk * uu);
        }
        __syncthreads();
        const f32x4 uu = reinterpret_cast<const f32x4 *>(su)[cg];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + ROWG * i;
            s[j][i] = s[j][i] + (bt * sk[r]) * uu;
        }
    };

#pragma unroll
    for (int j = 0; j < DEC_UNITS; ++j) {
        if (j >= nu) break;
        if (j + 1 < DEC_UNITS) fetch_state(j + 1);
#pragma unroll
        for (int jj = 0; jj < TOK_STAGED; ++jj) {
            if (jj >= len[j]) break;
            step(j, jj, xw[j][jj], xb[j][jj]);
        }
        for (int jj = TOK_STAGED; jj < len[j]; ++jj) {
            const int64_t row = (int64_t)(t0[j] + jj) * H + hh[j];
            step(j, jj, load_word(row), beta[row]);
        }
        // the next pair's state has had this pair's tokens to arrive: taking
        // it here keeps the optional stores below out of its wait
        if (j + 1 < DEC_UNITS) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) asm volatile("" ::"v"(s[j + 1][i]));
        }
        if (state_out) {
            f32x4 *W4 = reinterpret_cast<f32x4 *>(state_out + (u0 + j) * (int64_t)D * D);
#pragma unroll
            for (int i = 0; i < RPT; ++i) __builtin_nontemporal_store(s[j][i], &W4[(rg + ROWG * i) * (D / 4) + cg]);
        }
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
    if (T_tot <= 0) {   // no tokens: the state is committed unchanged
        if (state_out && state_out != state_in)
            return hipMemcpyAsync(state_out, state_in, sizeof(float) * (size_t)units * D * D, hipMemcpyDeviceToDevice,
                                  stream);
        return hipSuccess;
    }
    const dim3 grid((unsigned)((units + DEC_UNITS - 1) / DEC_UNITS));
    if (bf16)
        hipLaunchKernelGGL(kda_decode_tokens_kernel<bf16_t>, grid, dim3(DEC_THREADS), 0, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k),
                           static_cast<const bf16_t *>(v), g, beta, cu, num_tokens, state_in, state_out, H, T_tot,
                           units, static_cast<bf16_t *>(out));
    else
        hipLaunchKernelGGL(kda_decode_tokens_kernel<float>, grid, dim3(DEC_THREADS), 0, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(v), g, beta, cu, num_tokens, state_in, state_out, H, T_tot,
                           units, static_cast<float *>(out));
    return hipGetLastError();
}
