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
// (context-parallel pipeline with state stores), and inside a chunk the
// workgroup rebuilds the token states it needs in registers, then walks them
// backwards.
//
// Segments.  The gradient recurrence is linear in dS, as the forward one is
// in S (dS_{t-1} = Diag(alpha) (I - beta k k^T) (dS_t + q do^T)), so the
// sequences are cut into chunk-aligned segments that run side by side, as in
// the context-parallel forward: a summary pass takes each segment but a
// sequence's first from a zero gradient at its end to its start over the 128
// value columns, giving G^0; the segment's gradient transition R is the
// transpose of its forward transition M, which the forward pipeline's
// summaries already hold (the forward step is S_t = (I - beta k k^T) Diag(alpha)
// S_{t-1}, the gradient step its transpose, and a product of transposes in
// reverse order is the transpose of the product).  A reverse combine then
// gives the gradient entering every segment at its end, G(last) =
// d(final_state), G(s-1) = M_s^T G(s) + G^0_s, and the main pass runs every
// segment from there.
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
// head, block of 32 of the ncols columns), segments that are not a sequence's
// first; each wave runs its 8 columns on its own (no barrier).  seg_out:
// [num_segs][H][BD][ncols]: [G^0 | R] per segment for ncols = 2 BD, G^0 alone
// for ncols = BD (R is then the transpose of the forward transition M of the
// same segment: dS_{t-1} = Diag(alpha)(I - beta k k^T) dS_t is the transpose of
// the forward step's map, applied in the opposite order).
template <typename T>
__global__ __launch_bounds__(BWD_THREADS) void kda_backward_summary_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const T *__restrict__ dout, const int32_t *__restrict__ plan,
    int32_t num_segs, int32_t H, int32_t T_tot, int32_t ncols, float *__restrict__ seg_out)
{
    __shared__ __align__(16) float sv[BWD_THREADS / 64][3][BD];   // per wave: k, alpha, q
    const int ncb = ncols / BWD_BV;
    const int blk = blockIdx.x % ncb;
    const int64_t unit = blockIdx.x / ncb;
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
    float *dst = seg_out + ((int64_t)su * H + h) * BD * ncols;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<f32x2 *>(dst + (int64_t)(rg + 16 * i) * ncols + c0) = G[i];
}

// Work items (segment su, head h, column block blk) in the order
// item = (su H + h) NBLK + blk, walked with a stride of the grid (the scratch
// area belongs to the workgroup, not the item).  seg_dsend: [num_segs][H][BD][BD],
// the gradient entering each segment at its end.  part_vec: [NBLK][3][T_tot * H][BD]
// partial row sums (dq, dk, dg); part_beta: [NBLK][T_tot * H]; scratch:
// [gridDim.x][BWD_C / BWD_G + 1][BD][BWD_BV] floats; snaps: [chunks][H][BD][BD], the
// state at the start of global chunk chunk_off[n] + c for c >= 1 (c = 0 is the
// initial state).
//
// Each wave runs its 8 columns on its own, in the wave-level layout above.  Per
// chunk: a forward walk from the chunk's start state keeps u of every token (in
// LDS) and the state before every 4th token (in the scratch area, each lane's own
// values); then the chunk is walked backwards in groups of 4 tokens, whose 4
// states are rebuilt in registers from the group's stored state and the kept u
// (S = Diag(alpha) S + beta k u^T, no reduction).  A token's row sums (dq, dk, dg
// over the wave's columns) are reduced across the wave's four DPP rows so that
// each lane keeps 6 of the 3 x 128; after each group the four waves' sums meet in
// LDS and the workgroup adds them in wave order and writes its partials.
constexpr int BWD_G = 4;                  // tokens per reverse group (and per partial-sum batch)
constexpr int BWD_RED = 3 * BD;           // row sums per token and wave

__device__ __forceinline__ float perm32_sum(float a, float b) {   // lanes 0-31: a over lanes L, L+32; 32-63: b
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float perm16_sum(float a, float b) {   // even DPP rows: a over rows 2m, 2m+1; odd: b
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

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
    typedef typename Pair<T>::type Raw2;
    constexpr int NWV = BWD_THREADS / 64;
    __shared__ __align__(16) float tv[NWV][BWD_G][3][BD];       // per wave: k, alpha, q of a group's tokens
    __shared__ __align__(16) float su[NWV][BWD_C][8];            // per wave: u of the chunk's tokens
    __shared__ __align__(16) float red[NWV][BWD_G * BWD_RED];   // per wave: row sums of a group
    __shared__ float redb[NWV][BWD_G];                           // per wave: dbeta of a group

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rg = lane & 15, cg = lane >> 4;
    const int64_t rows_all = (int64_t)T_tot * H;
    // scratch: [checkpoint][wave][4][lane] f32x4, rows rg + 16 i of the lane's two columns
    f32x4 *scr = reinterpret_cast<f32x4 *>(scratch + (int64_t)blockIdx.x * (BWD_C / BWD_G + 1) * BD * BWD_BV) +
                 wave * 4 * 64 + lane;
    constexpr int CK = NWV * 4 * 64;                             // f32x4 per checkpoint
    const int64_t items = (int64_t)num_segs * H * BWD_NBLK;
    float *rw = red[wave];

    // a token's channel vectors (channels 2 lane, 2 lane + 1) to the wave's LDS
    // slot, read back as this lane's rows rg + 16 i (written and read by this
    // wave only, in order)
    auto put = [&](float *dst, float x0, float x1) {
        dst[chan_pos(2 * lane)] = x0;
        dst[chan_pos(2 * lane + 1)] = x1;
    };
    auto get = [&](const float *src, float r[8]) {
        *reinterpret_cast<f32x4 *>(r) = *reinterpret_cast<const f32x4 *>(src + 8 * rg);
        *reinterpret_cast<f32x4 *>(r + 4) = *reinterpret_cast<const f32x4 *>(src + 8 * rg + 4);
    };

  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int blk = (int)(item % BWD_NBLK);
    const int64_t unit = item / BWD_NBLK;                 // (segment, head)
    const int sg = (int)(unit / H), h = (int)(unit % H);
    const int n = plan[4 * sg];
    if (n < 0) continue;                                  // unused plan entry (uniform per workgroup)
    const int flags = plan[4 * sg + 3];
    const int cb = blk * BWD_BV + 8 * wave + 2 * cg;      // this lane's value columns cb, cb + 1
    const int t0 = min(max(cu[n], 0), T_tot);             // the sequence
    const int ts = min(max(plan[4 * sg + 1], t0), T_tot); // the segment: [ts, te), chunk-aligned in the sequence
    const int te = min(max(plan[4 * sg + 2], ts), T_tot);
    const int nch = (te - ts + BWD_C - 1) / BWD_C;
    const int64_t sbase = ((int64_t)n * H + h) * BD * BD;   // this (sequence, head) in [N, H, BD, BD]
    const float *gin = seg_dsend + unit * BD * BD;

    f32x2 dS[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) dS[i] = *reinterpret_cast<const f32x2 *>(gin + (int64_t)(rg + 16 * i) * BD + cb);

    for (int c = nch - 1; c >= 0; --c) {
        const int c0 = ts + c * BWD_C, Lc = min(BWD_C, te - c0);
        const int cs = (c0 - t0) / BWD_C;                 // chunk index within the sequence
        const float *src = cs ? snaps + ((int64_t)(chunk_off[n] + cs) * H + h) * BD * BD
                              : (initial_state ? initial_state + sbase : nullptr);
        f32x2 S[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            S[i] = src ? *reinterpret_cast<const f32x2 *>(src + (int64_t)(rg + 16 * i) * BD + cb) : f32x2{0.f, 0.f};

        // ---- forward over the chunk in groups of BWD_G tokens: u of every
        // token; the state before every group to the scratch area.  A group's
        // token vectors are loaded while the group before it runs, ahead of
        // that group's state store: vector memory operations complete in
        // order, so a load issued after a store could not be waited for
        // without waiting for the store.  Every step is branch-free (tokens
        // past the chunk's end are neutral: decay 1, write strength 0), so the
        // compiler counts the operations in flight exactly.
        // Two register sets in turn (groups taken in pairs, the group count
        // padded to even with neutral groups): a set loaded during one group
        // and read in the next would otherwise be copied at the loop's end,
        // and the copy waits for the load.
        struct FwdSet { Raw2 k[BWD_G], v[BWD_G]; f32x2 g[BWD_G]; float b[BWD_G]; };
        FwdSet fa, fb_;
        auto fetch_fwd = [&](int m, FwdSet &f) {
#pragma unroll
            for (int jj = 0; jj < BWD_G; ++jj) {
                const int64_t row = (int64_t)(c0 + min(m * BWD_G + jj, Lc - 1)) * H + h;
                f.k[jj] = *reinterpret_cast<const Raw2 *>(k + row * BD + 2 * lane);
                f.g[jj] = *reinterpret_cast<const f32x2 *>(g + row * BD + 2 * lane);
                f.v[jj] = *reinterpret_cast<const Raw2 *>(v + row * BD + cb);
                f.b[jj] = beta[row];
            }
            asm volatile("" ::: "memory");   // keep the loads here
        };
        auto store_state = [&](int m) {   // the state before token m * BWD_G (slot m; slot BWD_C / BWD_G is spare)
            f32x4 *sj = scr + m * CK;
#pragma unroll
            for (int p = 0; p < 4; ++p)
                sj[p * 64] = f32x4{S[2 * p][0], S[2 * p][1], S[2 * p + 1][0], S[2 * p + 1][1]};
        };
        auto fwd_group = [&](int m, const FwdSet &f) {
#pragma unroll
            for (int jj = 0; jj < BWD_G; ++jj) {
                const int j = m * BWD_G + jj;
                const bool ok = j < Lc;
                float *w = tv[wave][0][0];
                put(w, to_f(f.k[jj][0]), to_f(f.k[jj][1]));
                put(w + BD, ok ? __expf(f.g[jj][0]) : 1.f, ok ? __expf(f.g[jj][1]) : 1.f);
                __builtin_amdgcn_wave_barrier();
                float kr[8], ar[8];
                get(w, kr);
                get(w + BD, ar);
                __builtin_amdgcn_wave_barrier();
                float pa0 = 0.f, pa1 = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    S[i] *= ar[i];
                    pa0 += S[i][0] * kr[i];
                    pa1 += S[i][1] * kr[i];
                }
                const float u0 = to_f(f.v[jj][0]) - sum16(pa0), u1 = to_f(f.v[jj][1]) - sum16(pa1);
                if (rg == 0) *reinterpret_cast<f32x2 *>(&su[wave][j][2 * cg]) = f32x2{u0, u1};
                const float bt = ok ? f.b[jj] : 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float bk = bt * kr[i];
                    S[i][0] += bk * u0;
                    S[i][1] += bk * u1;
                }
            }
        };
        const int ngf = (Lc + 2 * BWD_G - 1) / (2 * BWD_G) * 2;     // groups, padded to even (<= BWD_C / BWD_G)
        fetch_fwd(0, fa);
        store_state(0);
        for (int m = 0; m < ngf; m += 2) {
            fetch_fwd(m + 1, fb_);
            fwd_group(m, fa);
            store_state(m + 1);
            fetch_fwd(min(m + 2, ngf - 1), fa);
            fwd_group(m + 1, fb_);
            store_state(m + 2);
        }
        __builtin_amdgcn_wave_barrier();

        // ---- backwards in groups of BWD_G tokens; a group's vectors and stored
        // state are loaded while the group before it is processed
        Raw2 gk[BWD_G], gq[BWD_G], gd[BWD_G];
        f32x2 gg_[BWD_G];
        float gb[BWD_G];
        f32x4 ck[4];
        auto fetch_group = [&](int m) {
#pragma unroll
            for (int jj = 0; jj < BWD_G; ++jj) {
                const int64_t row = (int64_t)(c0 + min(m * BWD_G + jj, Lc - 1)) * H + h;
                gk[jj] = *reinterpret_cast<const Raw2 *>(k + row * BD + 2 * lane);
                gg_[jj] = *reinterpret_cast<const f32x2 *>(g + row * BD + 2 * lane);
                gq[jj] = *reinterpret_cast<const Raw2 *>(q + row * BD + 2 * lane);
                gd[jj] = *reinterpret_cast<const Raw2 *>(dout + row * BD + cb);
                gb[jj] = beta[row];
            }
            const f32x4 *sj = scr + m * CK;                  // this lane's own stores: in order
#pragma unroll
            for (int p = 0; p < 4; ++p) ck[p] = sj[p * 64];
        };
        const int mtop = (Lc - 1) / BWD_G;
        fetch_group(mtop);
        for (int m = mtop; m >= 0; --m) {
            const int jl = m * BWD_G, ng = min(BWD_G, Lc - jl);
            f32x2 dd[BWD_G], Sp[BWD_G][8];
            float bb[BWD_G];
#pragma unroll
            for (int jj = 0; jj < BWD_G; ++jj) {
                float *w = tv[wave][jj][0];
                put(w, to_f(gk[jj][0]), to_f(gk[jj][1]));
                put(w + BD, __expf(gg_[jj][0]), __expf(gg_[jj][1]));
                put(w + 2 * BD, to_f(gq[jj][0]), to_f(gq[jj][1]));
                dd[jj] = f32x2{to_f(gd[jj][0]), to_f(gd[jj][1])};
                bb[jj] = gb[jj];
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                Sp[0][2 * p] = f32x2{ck[p][0], ck[p][1]};
                Sp[0][2 * p + 1] = f32x2{ck[p][2], ck[p][3]};
            }
            fetch_group(max(m - 1, 0));
            __builtin_amdgcn_wave_barrier();
            // the group's states before each token, from the stored one and the kept u
#pragma unroll
            for (int jj = 1; jj < BWD_G; ++jj) {
                if (jj < ng) {
                    float kr[8], ar[8];
                    get(tv[wave][jj - 1][0], kr);
                    get(tv[wave][jj - 1][1], ar);
                    const f32x2 u2 = *reinterpret_cast<const f32x2 *>(&su[wave][jl + jj - 1][2 * cg]);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float bk = bb[jj - 1] * kr[i];
                        Sp[jj][i][0] = Sp[jj - 1][i][0] * ar[i] + bk * u2[0];
                        Sp[jj][i][1] = Sp[jj - 1][i][1] * ar[i] + bk * u2[1];
                    }
                }
            }
#pragma unroll
            for (int jj = BWD_G - 1; jj >= 0; --jj) {
                if (jj < ng) {
                    const int j = jl + jj;
                    const int64_t row = (int64_t)(c0 + j) * H + h;
                    float kr[8], ar[8], qr[8];
                    get(tv[wave][jj][0], kr);
                    get(tv[wave][jj][1], ar);
                    get(tv[wave][jj][2], qr);
                    const f32x2 u2 = *reinterpret_cast<const f32x2 *>(&su[wave][j][2 * cg]);
                    const f32x2 d2 = dd[jj];
                    const float bt = bb[jj];
                    float px0 = 0.f, px1 = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        dS[i][0] += qr[i] * d2[0];                   // o = S^T q
                        dS[i][1] += qr[i] * d2[1];
                        px0 += dS[i][0] * kr[i];                     // dS^T k
                        px1 += dS[i][1] * kr[i];
                    }
                    const float x0 = sum16(px0), x1 = sum16(px1);
                    const float du0 = bt * x0, du1 = bt * x1;
                    if (rg == 0) *reinterpret_cast<f32x2 *>(dv_out + row * BD + cb) = f32x2{du0, du1};
                    float V[24];                                      // [dq | dk | dg] rows rg + 16 i, this lane's columns
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float a = ar[i], kr_ = kr[i], bk = bt * kr_;
                        const f32x2 sp = Sp[jj][i];
                        const f32x2 sb = sp * a;
                        const f32x2 sn = sb + bk * u2;
                        V[i] = sn[0] * d2[0] + sn[1] * d2[1];
                        V[8 + i] = bt * (dS[i][0] * u2[0] + dS[i][1] * u2[1]) - (sb[0] * du0 + sb[1] * du1);
                        const f32x2 dsb = f32x2{dS[i][0] - kr_ * du0, dS[i][1] - kr_ * du1};
                        V[16 + i] = a * (dsb[0] * sp[0] + dsb[1] * sp[1]);
                        dS[i] = dsb * a;
                    }
                    // sums over the wave's four DPP rows, scattered: lane cg keeps V[6 cg + e]
                    float W[12], X[6];
#pragma unroll
                    for (int e = 0; e < 12; ++e) W[e] = perm32_sum(V[e], V[e + 12]);
#pragma unroll
                    for (int e = 0; e < 6; ++e) X[e] = perm16_sum(W[e], W[e + 6]);
#pragma unroll
                    for (int e = 0; e < 6; ++e) {
                        const int ee = 6 * cg + e;                    // quantity ee / 8, row rg + 16 (ee % 8)
                        rw[jj * BWD_RED + (ee >> 3) * BD + rg + 16 * (ee & 7)] = X[e];
                    }
                    const float db = sum_rows4(x0 * u2[0] + x1 * u2[1]);
                    if (lane == 0) redb[wave][jj] = db;
                }
            }
            // the group's partial sums: the four waves added in order
            __syncthreads();
            for (int idx = threadIdx.x; idx < ng * BWD_RED; idx += BWD_THREADS) {
                float s = red[0][idx];
#pragma unroll
                for (int wv = 1; wv < NWV; ++wv) s += red[wv][idx];
                const int tok = idx / BWD_RED, rem = idx - tok * BWD_RED;
                const int qn = rem / BD, r = rem - qn * BD;
                const int64_t prow = (int64_t)(c0 + jl + tok) * H + h;
                part_vec[(((int64_t)blk * 3 + qn) * rows_all + prow) * BD + r] = s;
            }
            if ((int)threadIdx.x < ng) {
                float s = redb[0][threadIdx.x];
#pragma unroll
                for (int wv = 1; wv < NWV; ++wv) s += redb[wv][threadIdx.x];
                part_beta[(int64_t)blk * rows_all + (int64_t)(c0 + jl + threadIdx.x) * H + h] = s;
            }
            __syncthreads();
        }
    }

    if (dinit && (flags & SEG_FIRST)) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<f32x2 *>(dinit + sbase + (int64_t)(rg + 16 * i) * BD + cb) = dS[i];
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

// Scratch floats per workgroup of the main pass, and the most workgroups it
// launches (the item loop covers the rest): 512 x 144 KB of scratch at most.
extern "C" size_t kda_backward_scratch_floats_per_wg() { return (size_t)(kda::BWD_C / kda::BWD_G + 1) * kda::BD * kda::BWD_BV; }
extern "C" int32_t kda_backward_max_wgs() { return 512; }
extern "C" int32_t kda_backward_num_blocks() { return kda::BWD_NBLK; }

extern "C" hipError_t kda_launch_backward_summary(int bf16, const void *q, const void *k, const float *g,
                                                  const float *beta, const void *dout, const int32_t *plan,
                                                  int32_t num_segs, int32_t T_tot, int32_t H, int32_t ncols,
                                                  float *seg_out, hipStream_t stream)
{
    using namespace kda;
    if (ncols != BD && ncols != 2 * BD) return hipErrorInvalidValue;
    const int64_t grid = (int64_t)num_segs * H * (ncols / BWD_BV);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (bf16)
        hipLaunchKernelGGL(kda_backward_summary_kernel<bf16_t>, dim3((unsigned)grid), dim3(BWD_THREADS), 0, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k), g, beta,
                           static_cast<const bf16_t *>(dout), plan, num_segs, H, T_tot, ncols, seg_out);
    else
        hipLaunchKernelGGL(kda_backward_summary_kernel<float>, dim3((unsigned)grid), dim3(BWD_THREADS), 0, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k), g, beta,
                           static_cast<const float *>(dout), plan, num_segs, H, T_tot, ncols, seg_out);
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
