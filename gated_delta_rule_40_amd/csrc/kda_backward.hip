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
// and dbeta sum over columns.  So one work item is a (segment, head) and a
// block of BV = 32 value columns, with S and dS in registers; its row sums go
// to per-block partial buffers that a second kernel adds in a fixed order
// (deterministic).  The forward states are needed in reverse order: the
// state at every 32-token chunk start comes from the forward prefill kernel
// (snapshot mode), and inside a chunk the workgroup recomputes the 32 token
// states into its own scratch area, then walks them backwards.
//
// Segments.  The gradient recurrence is linear in dS, as the forward one is
// in S (dS_{t-1} = Diag(alpha) (I - beta k k^T) (dS_t + q do^T)), so the
// sequences are cut into chunk-aligned segments that run side by side, as in
// the context-parallel forward: a summary pass takes each segment but a
// sequence's first from a zero gradient at its end to its start over 128
// value columns plus 128 transition columns (identity at the end, do = 0),
// giving [G^0 | R]; a reverse combine then gives the gradient entering every
// segment at its end, G(last) = d(final_state), G(s-1) = R_s G(s) + G^0_s; and
// the main pass runs every segment from there.
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

// ---- wave-level layout.  A wave owns 8 columns: lane = rg + 16 cg holds rows
// rg + 16 i (i = 0..7) of columns 2 cg, 2 cg + 1.  A sum over the 128 rows
// is a sum over the 16 lanes of a DPP row (symmetric exchanges, so every lane
// ends with the same value); a sum over the wave's columns is a sum over its
// four DPP rows.  Token vectors go through a wave-private LDS area with
// channel c at (c mod 16) 8 + c / 16, so that a lane's 8 rows are contiguous.
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
__device__ __forceinline__ int chan_pos(int c) { return (c & 15) * 8 + (c >> 4); }

// Segment summaries of the gradient recurrence: one workgroup per (segment,
// head, block of 32 of the 128 + 128 columns), segments that are not a
// sequence's first; each wave runs its 8 columns on its own (no barrier).
// seg_out: [num_segs][H][BD][2 BD], [G^0 | R] per segment.
template <typename T>
__global__ __launch_bounds__(BWD_THREADS) void kda_backward_summary_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const T *__restrict__ dout, const int32_t *__restrict__ plan,
    int32_t num_segs, int32_t H, int32_t T_tot, float *__restrict__ seg_out)
{
    __shared__ __align__(16) float sv[BWD_THREADS / 64][3][BD];   // per wave: k, alpha, q
    constexpr int NB2 = 2 * BD / BWD_BV;
    const int blk = blockIdx.x % NB2;
    const int64_t unit = blockIdx.x / NB2;
    if (unit >= (int64_t)num_segs * H) return;
    const int su = (int)(unit / H), h = (int)(unit % H);
    if (plan[4 * su] < 0 || (plan[4 * su + 3] & SEG_FIRST)) return;
    const int ts = min(max(plan[4 * su + 1], 0), T_tot);
    const int te = min(max(plan[4 * su + 2], ts), T_tot);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rg = lane & 15, cg = lane >> 4;
    const int c0 = blk * BWD_BV + 8 * wave + 2 * cg;   // this lane's columns c0, c0 + 1 in [0, 2 BD)
    const bool trans = blk * BWD_BV >= BD;            // transition columns: identity at the end, do = 0
    float (*w)[BD] = sv[wave];
    f32x2 G[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = rg + 16 * i;
        G[i][0] = (trans && r == c0 - BD) ? 1.f : 0.f;
        G[i][1] = (trans && r == c0 + 1 - BD) ? 1.f : 0.f;
    }
    // the next token's vectors, one step ahead: channels 2 lane, 2 lane + 1 of
    // k, g, q, and this lane's two columns of dout (clamped rows: loads on every path)
    f32x2 nk, ng, nq, ndo;
    float nb;
    auto fetch = [&](int tt) {
        const int64_t row = (int64_t)tt * H + h;
        nk = load_pair(k + row * BD + 2 * lane);
        ng = *reinterpret_cast<const f32x2 *>(g + row * BD + 2 * lane);
        nq = load_pair(q + row * BD + 2 * lane);
        ndo = load_pair(dout + row * BD + (c0 & (BD - 1)));
        nb = beta[row];
    };
    if (te > ts) fetch(te - 1);
    for (int tt = te - 1; tt >= ts; --tt) {
        const f32x2 kk = nk, gg = ng, qq = nq, dd = trans ? f32x2{0.f, 0.f} : ndo;
        const float bt = nb;
        fetch(max(tt - 1, ts));
        // wave-private LDS: written and read by this wave only, in order
        w[0][chan_pos(2 * lane)] = kk[0];
        w[0][chan_pos(2 * lane + 1)] = kk[1];
        w[1][chan_pos(2 * lane)] = __expf(gg[0]);
        w[1][chan_pos(2 * lane + 1)] = __expf(gg[1]);
        w[2][chan_pos(2 * lane)] = qq[0];
        w[2][chan_pos(2 * lane + 1)] = qq[1];
        __builtin_amdgcn_wave_barrier();
        float kr[8], ar[8], qr[8];
        *reinterpret_cast<f32x4 *>(kr) = *reinterpret_cast<const f32x4 *>(&w[0][8 * rg]);
        *reinterpret_cast<f32x4 *>(kr + 4) = *reinterpret_cast<const f32x4 *>(&w[0][8 * rg + 4]);
        *reinterpret_cast<f32x4 *>(ar) = *reinterpret_cast<const f32x4 *>(&w[1][8 * rg]);
        *reinterpret_cast<f32x4 *>(ar + 4) = *reinterpret_cast<const f32x4 *>(&w[1][8 * rg + 4]);
        *reinterpret_cast<f32x4 *>(qr) = *reinterpret_cast<const f32x4 *>(&w[2][8 * rg]);
        *reinterpret_cast<f32x4 *>(qr + 4) = *reinterpret_cast<const f32x4 *>(&w[2][8 * rg + 4]);
        __builtin_amdgcn_wave_barrier();
        float px0 = 0.f, px1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            G[i][0] += qr[i] * dd[0];                   // o = S^T q
            G[i][1] += qr[i] * dd[1];
            px0 += G[i][0] * kr[i];                      // dS^T k
            px1 += G[i][1] * kr[i];
        }
        const float du0 = sum16(px0) * bt, du1 = sum16(px1) * bt;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            G[i][0] = (G[i][0] - kr[i] * du0) * ar[i];
            G[i][1] = (G[i][1] - kr[i] * du1) * ar[i];
        }
    }
    float *dst = seg_out + ((int64_t)su * H + h) * BD * (2 * BD);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<f32x2 *>(dst + (int64_t)(rg + 16 * i) * (2 * BD) + c0) = G[i];
}

// Work items (segment su, head h, column block blk) in the order
// item = (su H + h) NBLK + blk, walked with a stride of the grid (the scratch
// area belongs to the workgroup, not the item).  seg_dsend: [num_segs][H][BD][BD],
// the gradient entering each segment at its end.  part_vec: [NBLK][3][T_tot * H][BD]
// partial row sums (dq, dk, dg); part_beta: [NBLK][T_tot * H]; scratch:
// [gridDim.x][BWD_C][BD][BWD_BV]; snaps: [chunks][H][BD][BD], the state at the
// start of global chunk chunk_off[n] + c for c >= 1 (c = 0 is the initial state).
template <typename T>
__global__ __launch_bounds__(BWD_THREADS) void kda_backward_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *initial_state,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, const float *__restrict__ snaps,
    const T *__restrict__ dout, const int32_t *__restrict__ plan, int32_t num_segs,
    const float *__restrict__ seg_dsend, int32_t H, int32_t T_tot,
    float *__restrict__ scratch, float *__restrict__ part_vec, float *__restrict__ part_beta,
    float *__restrict__ dv_out, float *dinit)
{
    __shared__ float sq[BD], sk[BD], sa[BD];
    __shared__ float sv[BWD_BV], sdo[BWD_BV], su[BWD_BV], sx[BWD_BV];
    __shared__ f32x4 red_a[BWD_RG][BWD_CPR], red_x[BWD_RG][BWD_CPR];

    const int t = threadIdx.x;
    const int cg = t % BWD_CPR, rg = t / BWD_CPR;
    const int64_t rows_all = (int64_t)T_tot * H;
    float *scr = scratch + (int64_t)blockIdx.x * BWD_C * BD * BWD_BV;
    const int64_t items = (int64_t)num_segs * H * BWD_NBLK;

  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int blk = (int)(item % BWD_NBLK);
    const int64_t unit = item / BWD_NBLK;                 // (segment, head)
    const int sg = (int)(unit / H), h = (int)(unit % H);
    const int n = plan[4 * sg];
    if (n < 0) continue;                                  // unused plan entry (uniform per workgroup)
    const int flags = plan[4 * sg + 3];
    const int dv0 = blk * BWD_BV, c4 = dv0 + 4 * cg;
    const int t0 = min(max(cu[n], 0), T_tot);             // the sequence
    const int ts = min(max(plan[4 * sg + 1], t0), T_tot); // the segment: [ts, te), chunk-aligned in the sequence
    const int te = min(max(plan[4 * sg + 2], ts), T_tot);
    const int nch = (te - ts + BWD_C - 1) / BWD_C;
    const int64_t sbase = ((int64_t)n * H + h) * BD * BD;   // this (sequence, head) in [N, H, BD, BD]
    const float *gin = seg_dsend + unit * BD * BD;

    f32x4 S[BWD_RPT], dS[BWD_RPT], Sp[BWD_RPT];
#pragma unroll
    for (int i = 0; i < BWD_RPT; ++i) {
        const int r = rg + BWD_RG * i;
        dS[i] = *reinterpret_cast<const f32x4 *>(gin + (int64_t)r * BD + c4);
    }

    for (int c = nch - 1; c >= 0; --c) {
        const int c0 = ts + c * BWD_C, Lc = min(BWD_C, te - c0);
        const int cs = (c0 - t0) / BWD_C;                 // chunk index within the sequence
        const float *src = cs ? snaps + ((int64_t)(chunk_off[n] + cs) * H + h) * BD * BD
                              : (initial_state ? initial_state + sbase : nullptr);
#pragma unroll
        for (int i = 0; i < BWD_RPT; ++i) {
            const int r = rg + BWD_RG * i;
            S[i] = src ? *reinterpret_cast<const f32x4 *>(src + (int64_t)r * BD + c4) : zero4();
        }

        // ---- forward inside the chunk: scr[j] = state before token c0 + j
        // token vectors one step ahead, clamped rows (loads on every path)
        const int tc = min(t, BD - 1), vc = min(t, BWD_BV - 1);
        float nk, ng, nq, nv, ndo, nb;
        auto fetch = [&](int j) {
            const int64_t row = (int64_t)(c0 + j) * H + h;
            nk = to_f(k[row * BD + tc]);
            ng = g[row * BD + tc];
            nq = to_f(q[row * BD + tc]);
            nv = to_f(v[row * BD + dv0 + vc]);
            ndo = to_f(dout[row * BD + dv0 + vc]);
            nb = beta[row];
        };
        fetch(0);
        for (int j = 0; j < Lc; ++j) {
#pragma unroll
            for (int i = 0; i < BWD_RPT; ++i)
                *reinterpret_cast<f32x4 *>(scr + ((int64_t)j * BD + rg + BWD_RG * i) * BWD_BV + 4 * cg) = S[i];
            __syncthreads();                                   // token vectors free
            if (t < BD) {
                sk[t] = nk;
                sa[t] = __expf(ng);
            }
            if (t < BWD_BV) sv[t] = nv;
            const float bt = nb;
            fetch(min(j + 1, Lc - 1));
            __syncthreads();
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
        fetch(Lc - 1);
        f32x4 nSp[BWD_RPT];
        auto fetch_sp = [&](int j) {
#pragma unroll
            for (int i = 0; i < BWD_RPT; ++i)
                nSp[i] = *reinterpret_cast<const f32x4 *>(scr + ((int64_t)j * BD + rg + BWD_RG * i) * BWD_BV + 4 * cg);
        };
        fetch_sp(Lc - 1);                                      // this thread's own stores: in order
        for (int j = Lc - 1; j >= 0; --j) {
            const int64_t row = (int64_t)(c0 + j) * H + h;
#pragma unroll
            for (int i = 0; i < BWD_RPT; ++i) Sp[i] = nSp[i];
            __syncthreads();
            if (t < BD) {
                sq[t] = nq;
                sk[t] = nk;
                sa[t] = __expf(ng);
            }
            if (t < BWD_BV) {
                sv[t] = nv;
                sdo[t] = ndo;
            }
            const float bt = nb;
            fetch(max(j - 1, 0));
            fetch_sp(max(j - 1, 0));
            __syncthreads();
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

    if (dinit && (flags & SEG_FIRST)) {
#pragma unroll
        for (int i = 0; i < BWD_RPT; ++i) {
            const int r = rg + BWD_RG * i;
            *reinterpret_cast<f32x4 *>(dinit + sbase + (int64_t)r * BD + c4) = dS[i];
        }
    }
    __syncthreads();                                      // the next item reuses the token vectors
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

// Scratch floats per workgroup of the main pass, and the most workgroups it
// launches (the item loop covers the rest): 512 x 512 KB of scratch at most.
extern "C" size_t kda_backward_scratch_floats_per_wg() { return (size_t)kda::BWD_C * kda::BD * kda::BWD_BV; }
extern "C" int32_t kda_backward_max_wgs() { return 512; }
extern "C" int32_t kda_backward_num_blocks() { return kda::BWD_NBLK; }

extern "C" hipError_t kda_launch_backward_summary(int bf16, const void *q, const void *k, const float *g,
                                                  const float *beta, const void *dout, const int32_t *plan,
                                                  int32_t num_segs, int32_t T_tot, int32_t H, float *seg_out,
                                                  hipStream_t stream)
{
    using namespace kda;
    const int64_t grid = (int64_t)num_segs * H * (2 * BD / BWD_BV);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (bf16)
        hipLaunchKernelGGL(kda_backward_summary_kernel<bf16_t>, dim3((unsigned)grid), dim3(BWD_THREADS), 0, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k), g, beta,
                           static_cast<const bf16_t *>(dout), plan, num_segs, H, T_tot, seg_out);
    else
        hipLaunchKernelGGL(kda_backward_summary_kernel<float>, dim3((unsigned)grid), dim3(BWD_THREADS), 0, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k), g, beta,
                           static_cast<const float *>(dout), plan, num_segs, H, T_tot, seg_out);
    return hipGetLastError();
}

extern "C" hipError_t kda_launch_backward(int bf16, const void *q, const void *k, const void *v, const float *g,
                                          const float *beta, const float *init, const int32_t *cu,
                                          const int32_t *chunk_off, const float *snaps, const void *dout,
                                          const int32_t *plan, int32_t num_segs, const float *seg_dsend,
                                          int32_t N, int32_t T_tot, int32_t H, float *scratch,
                                          float *part_vec, float *part_beta, float *dq, float *dk, float *dv,
                                          float *dg, float *dbeta, float *dinit, hipStream_t stream)
{
    using namespace kda;
    const int64_t items = (int64_t)num_segs * H * BWD_NBLK;
    if (items <= 0) return hipSuccess;
    const int64_t grid = min(items, (int64_t)kda_backward_max_wgs());
    if (bf16)
        hipLaunchKernelGGL(kda_backward_kernel<bf16_t>, dim3((unsigned)grid), dim3(BWD_THREADS), 0, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k),
                           static_cast<const bf16_t *>(v), g, beta, init, cu, chunk_off, snaps,
                           static_cast<const bf16_t *>(dout), plan, num_segs, seg_dsend, H, T_tot, scratch,
                           part_vec, part_beta, dv, dinit);
    else
        hipLaunchKernelGGL(kda_backward_kernel<float>, dim3((unsigned)grid), dim3(BWD_THREADS), 0, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(v), g, beta, init, cu, chunk_off, snaps,
                           static_cast<const float *>(dout), plan, num_segs, seg_dsend, H, T_tot, scratch,
                           part_vec, part_beta, dv, dinit);
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
