// bf16 GEMMs on gfx950 MFMA for the shared-block projections.
//
// Every loop is "another Transformer pass" over the rows it recomputes
// (FlashLoop abstract, arxivdaily.com); in the lazy loops only the kept rows
// reach these kernels.  C = A[M, K] * W[N, K]^T with bf16 operands and fp32
// accumulation; epilogues fuse the residual add, SwiGLU and GELU.
//
// * Big-tile kernel (M >= 256, K % 128 == 0, N % 256 == 0): 256 x 256 x 64 tiles fed
//   by buffer loads straight into LDS; described at the kernel.
// * Tiled kernel (other M > 16): 128 x 128 x 32 tiles, 4 waves each owning 64 x 64 as
//   2 x 2 v_mfma_f32_32x32x16_bf16 tiles, LDS double buffering with one barrier
//   per k-step, rows padded to 80 bytes so the 16-byte operand reads of a wave
//   spread over the LDS banks.
// * Skinny kernels (decode, weight streaming; HBM bound).  The weights stream
//   straight from HBM into v_mfma_f32_16x16x32_bf16 B operands; the reduction
//   order over k is free, so A and B use the same permuted k order.
//   - Folded kernel (M <= 8): the 16 MFMA rows and columns are (K half, row)
//     pairs.  A row 8h + m holds activation row m over the h-th half of K, B
//     column 8h + n holds weight row n over the same half; the two diagonal 8x8
//     blocks of D summed are the product.  A tile is 8 weight rows, so there are
//     twice as many workgroups as with 16-row tiles, and the MFMA rows that M <= 8
//     would leave empty carry the second half of K instead of zeros.
//   - 16-row kernel (8 < M <= 16): one 16-row weight tile per workgroup.
//   In both, 8 waves split K and meet in LDS; every load of a wave covers 64
//   contiguous bytes of each of its rows.
#include <algorithm>
#include <atomic>

#include "lk_kernels.h"

namespace lk {

namespace {

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }
__device__ __forceinline__ float gelu_f(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// ---------------------------------------------------------------- tiled kernel
constexpr int BM = 128, BN = 128, BK = 32, LDK = BK + 8;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(const u16* __restrict__ A,
                                                         const u16* __restrict__ W, int M, int N,
                                                         int K, float* __restrict__ C,
                                                         u16* __restrict__ Obf) {
    __shared__ __attribute__((aligned(16))) u16 As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) u16 Bs[2][BN * LDK];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int l32 = lane & 31, kg = lane >> 5;
    const int row0 = blockIdx.y * BM;
    // rows of W loaded into the B tile
    const int wrows = (EPI == EPI_SWIGLU) ? 2 * N : N;

    uint4 ra[2], rb[2];
    int a_row[2], a_ch[2], b_wrow[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int c = tid + p * 256;
        const int rr = c >> 2;
        a_row[p] = rr;
        a_ch[p] = c & 3;
        int wr;
        if (EPI == EPI_SWIGLU) {
            const int blk = rr >> 5;
            wr = ((blk & 1) ? N : 0) + blockIdx.x * 64 + (blk >> 1) * 32 + (rr & 31);
        } else {
            wr = blockIdx.x * BN + rr;
        }
        b_wrow[p] = wr;
    }
    auto load = [&](int k0) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int gr = row0 + a_row[p];
            ra[p] = (gr < M) ? *(const uint4*)(A + (long long)gr * K + k0 + a_ch[p] * 8)
                             : make_uint4(0, 0, 0, 0);
            rb[p] = (b_wrow[p] < wrows) ? *(const uint4*)(W + (long long)b_wrow[p] * K + k0 + a_ch[p] * 8)
                                        : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            *(uint4*)&As[buf][a_row[p] * LDK + a_ch[p] * 8] = ra[p];
            *(uint4*)&Bs[buf][a_row[p] * LDK + a_ch[p] * 8] = rb[p];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][u][i] = 0.f;

    const int nk = K / BK;
    load(0);
    store(0);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        __syncthreads();
        if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 a[2], b[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
                a[t] = as_bf16x8(*(const uint4*)&As[cur][(wm * 64 + t * 32 + l32) * LDK + ks * 16 + kg * 8]);
#pragma unroll
            for (int u = 0; u < 2; ++u)
                b[u] = as_bf16x8(*(const uint4*)&Bs[cur][(wn * 64 + u * 32 + l32) * LDK + ks * 16 + kg * 8]);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], b[u], acc[t][u], 0, 0, 0);
        }
        if (kt + 1 < nk) store(cur ^ 1);
    }

    // epilogue: acc[t][u][i] = C[row0 + wm*64 + t*32 + 8*(i/4) + 4*kg + i%4][col(u) + l32]
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = row0 + wm * 64 + t * 32 + 8 * (i >> 2) + 4 * kg + (i & 3);
            if (r >= M) continue;
            if (EPI == EPI_SWIGLU) {
                const int col = blockIdx.x * 64 + wn * 32 + l32;
                if (col < N) Obf[(long long)r * N + col] = f2bf(silu_f(acc[t][0][i]) * acc[t][1][i]);
            } else {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int col = blockIdx.x * BN + wn * 64 + u * 32 + l32;
                    if (col >= N) continue;
                    const long long o = (long long)r * N + col;
                    if (EPI == EPI_STORE) C[o] = acc[t][u][i];
                    else if (EPI == EPI_ADD) C[o] = C[o] + acc[t][u][i];
                    else Obf[o] = f2bf(gelu_f(acc[t][u][i]));
                }
            }
        }
    }
}

// ---------------------------------------------------------------- skinny kernel
// NORM: the A operand is RMSNorm(X) * gain computed on the fly from float32 rows X:
// the kernel multiplies by bf16(X * gain), reduces the row sums of squares in the same
// pass and scales the result by 1 / sqrt(mean(X^2) + eps) in the epilogue.
template <int EPI, int J, bool NORM>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(const u16* __restrict__ A, const float* __restrict__ X,
                                                          const u16* __restrict__ gain, float eps,
                                                          const u16* __restrict__ W, int M, int N,
                                                          int K, float* __restrict__ C,
                                                          u16* __restrict__ Obf) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    __shared__ f32x4 red[8][64][DUAL ? 2 : 1];
    __shared__ float ssq[8][64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c16 = lane & 15, grp = lane >> 4;
    const int n = blockIdx.x * 16 + c16;
    constexpr int CH = 32 * J;  // k per chunk (4 lane groups x 8J)
    const int nch = K / CH;
    const int cb = w * nch / 8, ce = (w + 1) * nch / 8;
    const bool nvalid = n < N;
    const u16* w0 = W + (long long)(nvalid ? n : 0) * K;
    const u16* w1 = W + (long long)(nvalid ? N + n : 0) * K;
    const bool mvalid = c16 < M;
    const u16* ar = A + (long long)(mvalid ? c16 : 0) * K;
    const float* xr = X + (long long)(mvalid ? c16 : 0) * K;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
    for (int c = cb; c < ce; ++c) {
        const int k0 = c * CH + grp * 8 * J;
        uint4 wv[J], av[J], wv1[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            wv[j] = *(const uint4*)(w0 + k0 + j * 8);
            if (DUAL) wv1[j] = *(const uint4*)(w1 + k0 + j * 8);
            if (!NORM) av[j] = mvalid ? *(const uint4*)(ar + k0 + j * 8) : make_uint4(0, 0, 0, 0);
        }
        if (NORM) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                if (!mvalid) {
                    av[j] = make_uint4(0, 0, 0, 0);
                    continue;
                }
                const float4 xa = *(const float4*)(xr + k0 + j * 8);
                const float4 xb = *(const float4*)(xr + k0 + j * 8 + 4);
                const uint4 gv = *(const uint4*)(gain + k0 + j * 8);
                const float xs[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
                const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
                uint32_t o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    ss += xs[2 * q] * xs[2 * q] + xs[2 * q + 1] * xs[2 * q + 1];
                    o[q] = pack_bf2(xs[2 * q] * __uint_as_float(gw[q] << 16),
                                    xs[2 * q + 1] * __uint_as_float(gw[q] & 0xFFFF0000u));
                }
                av[j] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[j]), as_bf16x8(wv[j]), acc0, 0, 0, 0);
            if (DUAL)
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[j]), as_bf16x8(wv1[j]), acc1, 0, 0, 0);
        }
    }
    red[w][lane][0] = acc0;
    if (DUAL) red[w][lane][DUAL ? 1 : 0] = acc1;
    if (NORM) ssq[w][lane] = ss;
    __syncthreads();
    if (w != 0) return;
    f32x4 s0 = red[0][lane][0], s1 = DUAL ? red[0][lane][DUAL ? 1 : 0] : s0;
#pragma unroll
    for (int ww = 1; ww < 8; ++ww) {
        s0 += red[ww][lane][0];
        if (DUAL) s1 += red[ww][lane][DUAL ? 1 : 0];
    }
    // acc lane l: D[row = (l/16)*4 + i][col = l%16]
    float inv[4] = {1.f, 1.f, 1.f, 1.f};
    if (NORM) {
        // row m's partial sums sit in lanes m, m+16, m+32, m+48 of every wave
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = grp * 4 + i;
            float t = 0.f;
            for (int ww = 0; ww < 8; ++ww)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) t += ssq[ww][m + 16 * gq];
            inv[i] = 1.0f / sqrtf(t / (float)K + eps);
        }
    }
    if (!nvalid) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = grp * 4 + i;
        if (m >= M) continue;
        const long long o = (long long)m * N + n;
        const float v0 = s0[i] * inv[i];
        if (EPI == EPI_STORE) C[o] = v0;
        else if (EPI == EPI_ADD) C[o] = C[o] + v0;
        else if (EPI == EPI_SWIGLU) Obf[o] = f2bf(silu_f(v0) * (s1[i] * inv[i]));
        else Obf[o] = f2bf(gelu_f(v0));
    }
}


typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- folded skinny kernel
// Requires M <= 8 and K % 64 == 0.  Wave w takes the 32-element k chunks c = w, w + 8,
// ... of each half, NL chunks per batch of loads.
//
// PK (lane-packed operands, the decode products): W is the float16 decode copy of the
// weights, A float16 in the same lane-packed order (one rounding of the float32 value),
// and the 16-bit outputs (xg_out, Obf) are written that way; otherwise A, W and the
// outputs are bf16, row-major.
// NORM (RMSNorm folded in): A holds x * gain and ps_in [nparts][8] partial sums of x^2
// per row; the product is scaled by 1 / sqrt(sum / K + eps).
// PREP (with EPI_ADD): besides x += A W^T (+ add_vec), write what the next NORM
// product needs: xg_out = x * next_gain and, per workgroup, the row sums of x^2 over
// its 8 columns into ps_out [N / 8][8].
template <int EPI, int NL, bool NORM, bool PREP, bool PK, bool LIVE>
__global__ __launch_bounds__(512) void gemm_fold_kernel(const u16* __restrict__ A, const u16* __restrict__ W,
                                                        int M, int N, int K, float* __restrict__ C,
                                                        u16* __restrict__ Obf, FoldIO io) {
    if (LIVE && *io.live == 0) return;  // no sequence left in the loops
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    constexpr int NWV = 8;
    __shared__ f32x4 red[NWV][64][DUAL ? 2 : 1];
    __shared__ float s_inv[8];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c16 = lane & 15, grp = lane >> 4;
    const int h = c16 >> 3, r8 = c16 & 7;
    const int Kh = K >> 1, nch = Kh >> 5;
    const int n = blockIdx.x * 8 + r8;  // grid = N / 8 (N % 8 == 0)
    // PK: operands in the lane-packed order (chunk c of tile t at ((t nch + c) 64 + lane) 8)
    const u16* w0 = PK ? W + ((long long)blockIdx.x * nch * 64 + lane) * 8 : W + (long long)n * K + h * Kh + grp * 8;
    const u16* w1 = PK ? W + ((long long)(N / 8 + blockIdx.x) * nch * 64 + lane) * 8
                       : W + (long long)(N + n) * K + h * Kh + grp * 8;
    const int wstep = PK ? 512 : 32;  // elements between consecutive chunks
    const bool mvalid = r8 < M;
    const u16* ar = PK ? A + lane * 8 : A + (long long)(mvalid ? r8 : 0) * K + h * Kh + grp * 8;
    // The epilogue's inputs (partial sums of x^2 for the norm, the residual rows, the
    // added vector and the next norm's gain) are loaded before the weight stream so that
    // they do not cost a memory round trip after it.
    constexpr int PSR = 8;  // partial sums held in registers per lane (nparts <= 512)
    float ps_pre[PSR];
    const bool norm_wave = NORM && w < M;
    if (norm_wave) {
#pragma unroll
        for (int q = 0; q < PSR; ++q) {
            const int p = lane + 64 * q;
            ps_pre[q] = p < io.nparts ? io.ps_in[p * 8 + w] : 0.f;
        }
    }
    const bool out_lane = grp < 2 && c16 < 8;
    const int col = blockIdx.x * 8 + (c16 & 7);
    float c_pre[4] = {0.f, 0.f, 0.f, 0.f};
    float r_pre[4] = {0.f, 0.f, 0.f, 0.f};
    float addv = 0.f, gainv = 0.f;
    if (EPI == EPI_ADD && w == 0 && out_lane) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = (grp & 1) * 4 + i;
            if (m < M) c_pre[i] = C[(long long)m * N + col];
            if (PREP && io.add_rows && m < M) r_pre[i] = io.add_rows[(long long)m * N + col];
        }
        if (PREP && io.add_vec) addv = bf2f(io.add_vec[col]);
        if (PREP) gainv = bf2f(io.next_gain[col]);
    }
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    // float16 operands on the lane-packed path, bf16 on the row-major one
    auto mma = [](uint4 a, uint4 b, f32x4 c) {
        if constexpr (PK)
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                          0, 0, 0);
        else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
    };
    for (int c0 = w; c0 < nch; c0 += NWV * NL) {
        uint4 wv[NL], wv1[NL], av[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int c = c0 + j * NWV;
            const bool ok = c < nch;
            wv[j] = ok ? *(const uint4*)(w0 + (long long)c * wstep) : make_uint4(0, 0, 0, 0);
            if (DUAL) wv1[j] = ok ? *(const uint4*)(w1 + (long long)c * wstep) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int c = c0 + j * NWV;
            const bool ok = c < nch && mvalid;
            av[j] = ok ? *(const uint4*)(ar + (long long)c * wstep) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            acc0 = mma(av[j], wv[j], acc0);
            if (DUAL) acc1 = mma(av[j], wv1[j], acc1);
        }
    }
    if (norm_wave) {  // wave w: row w's sum of squares, partials in a fixed order
        float t = 0.f;
#pragma unroll
        for (int q = 0; q < PSR; ++q) t += ps_pre[q];
        for (int p = lane + 64 * PSR; p < io.nparts; p += 64) t += io.ps_in[p * 8 + w];
        t = wave_sum(t);
        if (lane == 0) s_inv[w] = 1.0f / sqrtf(t / (float)K + io.eps);
    }
    red[w][lane][0] = acc0;
    if (DUAL) red[w][lane][DUAL ? 1 : 0] = acc1;
    __syncthreads();
    if (w != 0) return;
    f32x4 s0 = red[0][lane][0], s1 = DUAL ? red[0][lane][DUAL ? 1 : 0] : s0;
#pragma unroll
    for (int ww = 1; ww < NWV; ++ww) {
        s0 += red[ww][lane][0];
        if (DUAL) s1 += red[ww][lane][DUAL ? 1 : 0];
    }
    // lane holds D[row 4 grp + i][col c16]; rows 8..15 and columns 8..15 are the second
    // K half: lane l (grp < 2, c16 < 8) adds lane l + 40 (rows +8, columns +8).
    f32x4 o0, o1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o0[i] = __shfl(s0[i], (lane + 40) & 63);
        if (DUAL) o1[i] = __shfl(s1[i], (lane + 40) & 63);
    }
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = (grp & 1) * 4 + i;
        if (!out_lane || m >= M) continue;
        const long long o = (long long)m * N + col;
        const float inv = NORM ? s_inv[m] : 1.f;
        const float v0 = (s0[i] + o0[i]) * inv;
        if (EPI == EPI_STORE) {
            C[o] = v0;
        } else if (EPI == EPI_ADD) {
            float x = c_pre[i] + v0;
            if (PREP && io.x_save) io.x_save[o] = x;
            if (PREP && io.add_rows) x = x + r_pre[i];
            if (PREP && io.add_vec) x = x + addv;
            C[o] = x;
            if (PREP) {
                if (PK) {
                    io.xg_out[pk_index(m, col, N)] = f2h_bits(x * gainv);
                } else {
                    io.xg_out[o] = f2bf(x * gainv);
                }
                sq[i] = x * x;
            }
        } else {
            const float y = EPI == EPI_SWIGLU ? silu_f(v0) * ((s1[i] + o1[i]) * inv) : gelu_f(v0);
            if (PK) {
                Obf[pk_index(m, col, N)] = f2h_bits(y);
            } else {
                Obf[o] = f2bf(y);
            }
        }
    }
    if (PREP) {
        // sum the 8 columns of this workgroup: lanes c16 = 0..7 of the same grp
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int off = 1; off < 8; off <<= 1) sq[i] += __shfl_xor(sq[i], off);
        if (out_lane && c16 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) io.ps_out[blockIdx.x * 8 + grp * 4 + i] = sq[i];
    }
}

template <int EPI, bool NORM, bool PREP, bool PK = false>
void launch_fold(const u16* A, const u16* W, int M, int N, int K, float* c, u16* out_bf, const FoldIO& io,
                 hipStream_t st) {
    // one batch of loads per wave at K = 2048 (4 chunks) and K = 5632 (11 chunks)
    const int per_wave = (K / 64 + 7) / 8;
    dim3 grid(N / 8);
    if (io.live && per_wave > 4)
        hipLaunchKernelGGL((gemm_fold_kernel<EPI, 11, NORM, PREP, PK, true>), grid, dim3(512), 0, st, A, W, M, N, K, c, out_bf, io);
    else if (io.live)
        hipLaunchKernelGGL((gemm_fold_kernel<EPI, 4, NORM, PREP, PK, true>), grid, dim3(512), 0, st, A, W, M, N, K, c, out_bf, io);
    else if (per_wave > 4)
        hipLaunchKernelGGL((gemm_fold_kernel<EPI, 11, NORM, PREP, PK, false>), grid, dim3(512), 0, st, A, W, M, N, K, c, out_bf, io);
    else
        hipLaunchKernelGGL((gemm_fold_kernel<EPI, 4, NORM, PREP, PK, false>), grid, dim3(512), 0, st, A, W, M, N, K, c, out_bf, io);
}

// The decode copy of a bf16 weight matrix: float16 in the lane-packed order.  A bf16
// value converts exactly when its magnitude lies in [2^-17, 65504] (float16 has three
// more mantissa bits; below 2^-14 it keeps 2^-24 steps); smaller magnitudes round to
// the nearest 2^-24 step (an error below 3e-8), larger ones become inf.
__global__ void pack_rows_kernel(const u16* __restrict__ W, long long rows, int K, u16* __restrict__ Wp) {
    const long long n8 = rows * K / 8;  // 16-byte pieces
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n8; i += (long long)gridDim.x * blockDim.x) {
        const long long row = i / (K / 8);
        const int k = (int)(i % (K / 8)) * 8;
        const uint4 v = *(const uint4*)(W + row * K + k);
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            o[t] = pack_h2(__uint_as_float(wv[t] << 16), __uint_as_float(wv[t] & 0xFFFF0000u));
        *(uint4*)(Wp + pk_index((int)row, k, K)) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

bool fold_ok(int M, int N, int K) { return M <= 8 && K % 64 == 0 && N % 8 == 0; }

template <int EPI, bool NORM>
void launch_skinny(const u16* A, const float* X, const u16* gain, float eps, const u16* W, int M, int N, int K,
                   float* c, u16* out_bf, hipStream_t st) {
    if (!NORM && fold_ok(M, N, K)) {
        launch_fold<EPI, false, false>(A, W, M, N, K, c, out_bf, FoldIO{}, st);
        return;
    }
    dim3 grid((N + 15) / 16);
    if (K % 128 == 0)
        hipLaunchKernelGGL((gemm_skinny_kernel<EPI, 4, NORM>), grid, dim3(512), 0, st, A, X, gain, eps, W, M, N, K, c, out_bf);
    else if (K % 64 == 0)
        hipLaunchKernelGGL((gemm_skinny_kernel<EPI, 2, NORM>), grid, dim3(512), 0, st, A, X, gain, eps, W, M, N, K, c, out_bf);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<EPI, 1, NORM>), grid, dim3(512), 0, st, A, X, gain, eps, W, M, N, K, c, out_bf);
}


// ---------------------------------------------------------------- big-tile kernel
// 256 x 256 workgroup tiles stepped 64 deep in k, 4 waves as 2 x 2, each wave 128 x 128
// as 4 x 4 v_mfma_f32_32x32x16_bf16 tiles (256 accumulators per lane, one wave per SIMD).
// Operands reach LDS by buffer loads with the LDS bit (16 bytes per lane, no register
// staging): a tile row is 64 bf16 = one 128-byte line, one load instruction moves 8
// whole rows, and the k offset rides in the scalar offset, so a load costs one M0 move.
// Two LDS stages of 64 KB: the next slab streams in while the current one is consumed.
// Within a stage, 16-byte chunk c of row r sits at slot c ^ f(r), f(r) = (r % 8) ^ (r / 8 % 2):
// the LDS serves a 16-byte read 16 lanes at a time over 64 banks, and the 16 rows read by
// 16 consecutive lanes cover every (row parity, slot) pair once, so they land in distinct
// banks.  The k loop is unrolled over the two stages (stage indices are compile-time,
// which keeps the compiler's LDS-DMA tracking exact), the LDS reads of the next k-slice
// are interleaved with the MFMAs of the current one, and there is one barrier per slab.
// The workgroup is persistent over tiles, XCD by XCD, grouped 8 M-tiles tall; the first
// two slabs of its next tile go out as soon as each stage is free, before the current
// tile's epilogue, so the epilogue's stores overlap the next tile's first loads.  Rows
// past M load as zeros and are not stored (buffer range checks).  SwiGLU: the 256 W rows
// of a tile are [gate 0..63 | up 0..63 | gate 64..127 | up 64..127] of 128 output
// columns, so each wave holds gate and up of its 64 output columns.
// Requires K % 128 == 0 and N % 256 == 0 (SwiGLU: N % 128 == 0).
constexpr int GB_M = 256, GB_N = 256, GB_K = 64, GB_STAGE = (GB_M + GB_N) * GB_K;

// Compute units of the current device (cached per device).
int cu_count() {
    static std::atomic<int> n[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!n[dev]) {
        int c = 0;
        n[dev] = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c >= 8 ? c : 256;
    }
    return n[dev];
}
__shared__ __attribute__((aligned(1024))) u16 gb_s0[GB_STAGE];
__shared__ __attribute__((aligned(1024))) u16 gb_s1[GB_STAGE];
typedef __attribute__((address_space(3))) void lds_void;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void bare_barrier() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
template <int U>
__device__ __forceinline__ u16* gb_stage() { return U == 0 ? gb_s0 : gb_s1; }

// LDS slot permutation of the 16-byte chunks of stage row r.
__device__ __forceinline__ int gb_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Buffer resources of the A and W rows of one tile and this lane's byte offsets.
struct GbSrc {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t va[8], vb[8];
};

// One 64-deep slab into a stage: wave ws moves 1 KB blocks ws + 4q of A and of W.
__device__ __forceinline__ void gb_issue(u16* st, const GbSrc& d, int k0, int ws) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (lds_void*)(st + (ws + 4 * q) * 512), 16, d.va[q], k0 * 2, 0, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rb, (lds_void*)(st + GB_M * GB_K + (ws + 4 * q) * 512), 16, d.vb[q],
                                                 k0 * 2, 0, 0);
}
// Operands of k-slice c (chunk index 0..7 = 16-element group incl. the lane's k half).
// Read order fa[0], fb[0..3], fa[1..3]: the order the MFMAs of the slice consume them.
__device__ __forceinline__ void gb_read(const u16* st, bf16x8 (&fa)[4], bf16x8 (&fb)[4], int wm, int wn, int l32,
                                        int c) {
    auto ra = [&](int i) {
        const int r = wm * 128 + 32 * i + l32;
        fa[i] = as_bf16x8(*(const uint4*)(st + r * GB_K + ((c ^ gb_swz(r)) * 8)));
    };
    ra(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = wn * 128 + 32 * j + l32;
        fb[j] = as_bf16x8(*(const uint4*)(st + GB_M * GB_K + r * GB_K + ((c ^ gb_swz(r)) * 8)));
    }
#pragma unroll
    for (int i = 1; i < 4; ++i) ra(i);
}
__device__ __forceinline__ void gb_mma(f32x16 (&acc)[4][4], const bf16x8 (&fa)[4], const bf16x8 (&fb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}
// scheduling: the eight LDS reads of the next k-slice go out one per MFMA over the
// first half of the 16 MFMAs of a group, so each has at least eight MFMAs (about 256
// cycles) to land before the next group needs it
__device__ __forceinline__ void gb_sched_reads() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // MFMA
}

// One slab in stage U.  On entry x holds k-slice 0 of the slab.  NEXT: another slab
// follows in stage U ^ 1 (wait for it, barrier, read its k-slice 0 into x); DMA: once
// every wave is past that barrier, refill stage U with slab k0 of the operands in dsrc
// (the slab after next, or the first slab of the next tile).
template <int U, bool NEXT, bool DMA>
__device__ __forceinline__ void gb_slab(f32x16 (&acc)[4][4], bf16x8 (&xa)[4], bf16x8 (&xb)[4], bf16x8 (&ya)[4],
                                        bf16x8 (&yb)[4], const GbSrc& dsrc, int k0, int ws, int wm, int wn,
                                        int l32, int kg) {
    gb_read(gb_stage<U>(), ya, yb, wm, wn, l32, 2 + kg);
    gb_mma(acc, xa, xb);
    gb_sched_reads();
    gb_read(gb_stage<U>(), xa, xb, wm, wn, l32, 4 + kg);
    gb_mma(acc, ya, yb);
    gb_sched_reads();
    gb_read(gb_stage<U>(), ya, yb, wm, wn, l32, 6 + kg);
    gb_mma(acc, xa, xb);
    gb_sched_reads();
    if (NEXT) {
        wait_vmcnt<0>();  // this wave's part of the next slab is in LDS
        bare_barrier();   // ... and every wave's; every wave is done reading stage U
        if (DMA) gb_issue(gb_stage<U>(), dsrc, k0, ws);
        gb_read(gb_stage<U ^ 1>(), xa, xb, wm, wn, l32, kg);
    }
    gb_mma(acc, ya, yb);
    if (NEXT) {
        if (DMA) {  // the 16 slab loads one per MFMA, the 8 LDS reads one per two
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // buffer load
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // buffer load
            }
        } else {
            gb_sched_reads();
        }
    }
}

// Tile t of the persistent order: groups of 8 M-tiles, N-tiles inside a group.
struct GbTile {
    int tm, tn;
};
__device__ __forceinline__ GbTile gb_tile_at(int t, int tiles_m, int tiles_n) {
    constexpr int GROUP = 8;
    const int group_size = GROUP * tiles_n;
    const int gid = t / group_size, first_m = gid * GROUP;
    const int gm = min(tiles_m - first_m, GROUP);
    return {first_m + (t % group_size) % gm, (t % group_size) / gm};
}

// Buffer resource over `rows` rows of `pitch` bytes from base: loads past the end return
// zeros and stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gb_rows_rsrc(const void* base, int rows, int pitch) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, rows * pitch, 0x00020000);
}

// Operand resources of tile (tm, tn); the lane offsets in va / vb do not depend on the tile.
template <bool DUAL>
__device__ __forceinline__ void gb_src_rsrc(GbSrc& d, const u16* A, const u16* W, int M, int N, int K, int tm,
                                            int tn) {
    const int row0 = tm * GB_M;
    d.ra = gb_rows_rsrc(A + (long long)row0 * K, min(M - row0, GB_M), K * 2);
    const long long wrow0 = DUAL ? (long long)tn * 128 : (long long)tn * GB_N;
    const int wspan = DUAL ? N + 128 : GB_N;  // W rows the tile reaches from wrow0
    d.rb = gb_rows_rsrc(W + wrow0 * K, wspan, K * 2);
}

// x * sigmoid(x) from the hardware base-2 exponential and reciprocal (about 1 ulp each;
// the product is rounded to bf16).
__device__ __forceinline__ float silu_fast(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// Epilogue of tile (tm, tn): acc[i][j][e] is C[row0 + wm*128 + 32 i + 8 (e/4) + 4 kg + e%4][col(j) + l32].
// Every access goes through a buffer resource over the tile's valid rows.
template <int EPI>
__device__ __forceinline__ void gb_epilogue(const f32x16 (&acc)[4][4], float* __restrict__ C, u16* __restrict__ Obf,
                                            int M, int N, int tm, int tn, int wm, int wn, int l32, int kg) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    const int row0 = tm * GB_M, rows = min(M - row0, GB_M);
    // byte offset of row 32 i + 8 (e/4) + e%4 of this lane's (wm, kg) rows
    auto roff = [&](int i, int e, int esz) { return (32 * i + 8 * (e >> 2) + (e & 3)) * N * esz; };
    if (DUAL) {
        const __amdgpu_buffer_rsrc_t ro = gb_rows_rsrc(Obf + (long long)row0 * N, rows, N * 2);
        const int base = ((wm * 128 + 4 * kg) * N + tn * 128 + wn * 64 + l32) * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int o = base + roff(i, e, 2);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    __builtin_amdgcn_raw_buffer_store_b16(f2bf(silu_fast(acc[i][j][e]) * acc[i][j + 2][e]), ro,
                                                          o + 64 * j, 0, 0);
            }
        return;
    }
    const __amdgpu_buffer_rsrc_t rc = gb_rows_rsrc(C + (long long)row0 * N, rows, N * 4);
    const int base = ((wm * 128 + 4 * kg) * N + tn * GB_N + wn * 128 + l32) * 4;
    if (EPI == EPI_ADD) {
        // residual add, software-pipelined over the four 32-row groups: the 64 loads of
        // group i + 1 are issued before the stores of group i
        float cv[2][16][4];
        auto load_group = [&](int i, float (&dst)[16][4]) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    dst[e][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                                              rc, base + roff(i, e, 4) + 128 * j, 0, 0));
        };
        load_group(0, cv[0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i + 1 < 4) load_group(i + 1, cv[(i + 1) & 1]);
#pragma unroll
            for (int e = 0; e < 16; ++e)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(cv[i & 1][e][j] + acc[i][j][e]),
                                                          rc, base + roff(i, e, 4) + 128 * j, 0, 0);
        }
    } else if (EPI == EPI_STORE) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][e]), rc,
                                                          base + roff(i, e, 4) + 128 * j, 0, 0);
    } else {  // GELU to bf16
        const __amdgpu_buffer_rsrc_t ro = gb_rows_rsrc(Obf + (long long)row0 * N, rows, N * 2);
        const int obase = base / 2;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __builtin_amdgcn_raw_buffer_store_b16(f2bf(gelu_f(acc[i][j][e])), ro,
                                                          obase + roff(i, e, 2) + 64 * j, 0, 0);
    }
}

// Persistent over tiles: workgroup b stays on XCD b % 8 and takes that XCD's share of
// the tiles (a contiguous range of the tile order) in turn, so a CU goes from one tile's
// epilogue straight to the next tile's loads, and CUs drift out of step instead of all
// storing at once.
template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_big_kernel(const u16* __restrict__ A, const u16* __restrict__ W,
                                                          int M, int N, int K, float* __restrict__ C,
                                                          u16* __restrict__ Obf, int tiles_m, int tiles_n) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    const int ntiles = tiles_m * tiles_n;
    const int per_xcd = (ntiles + 7) / 8;
    const int xcd = blockIdx.x % 8, slots = gridDim.x / 8;
    int local = blockIdx.x / 8;
    if (local >= per_xcd || xcd * per_xcd + local >= ntiles) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int ws = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = ws >> 1, wn = ws & 1, l32 = lane & 31, kg = lane >> 5;
    GbSrc src;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int r = 8 * (ws + 4 * q) + lane / 8;  // tile row of this lane's 16 bytes
        const int c = (lane % 8) ^ gb_swz(r);       // the chunk that lands in slot lane % 8
        src.va[q] = (uint32_t)(r * K * 2 + c * 16);
        int wr = r;
        if (DUAL) {
            const int h = r >> 6;  // 0: gate lo, 1: up lo, 2: gate hi, 3: up hi
            wr = ((h & 1) ? N : 0) + (h >> 1) * 64 + (r & 63);
        }
        src.vb[q] = (uint32_t)(wr * K * 2 + c * 16);
    }
    GbTile tile = gb_tile_at(xcd * per_xcd + local, tiles_m, tiles_n);
    gb_src_rsrc<DUAL>(src, A, W, M, N, K, tile.tm, tile.tn);
    gb_issue(gb_s0, src, 0, ws);
    gb_issue(gb_s1, src, GB_K, ws);
    const int ns = K / GB_K;  // even, >= 2
    for (bool first = true;; first = false) {
        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
        if (first) wait_vmcnt<16>();  // slab 0 is in
        else wait_vmcnt<0>();         // slabs 0 and 1 (and the last epilogue's stores)
        bare_barrier();
        bf16x8 xa[4], xb[4], ya[4], yb[4];
        gb_read(gb_s0, xa, xb, wm, wn, l32, kg);
        int s = 0;
        for (; s < ns - 2; s += 2) {
            gb_slab<0, true, true>(acc, xa, xb, ya, yb, src, (s + 2) * GB_K, ws, wm, wn, l32, kg);
            gb_slab<1, true, true>(acc, xa, xb, ya, yb, src, (s + 3) * GB_K, ws, wm, wn, l32, kg);
        }
        // the next tile of this workgroup: its slab 0 goes into stage 0 as soon as every
        // wave is done with it, its slab 1 into stage 1 after the last slab.  Without a
        // next tile the loads go through empty resources: no memory access, and the
        // zeros they leave in the stages are never read.
        const int nlocal = local + slots;
        const bool more = nlocal < per_xcd && xcd * per_xcd + nlocal < ntiles;
        GbSrc nsrc = src;
        const GbTile ntile = gb_tile_at(more ? xcd * per_xcd + nlocal : 0, tiles_m, tiles_n);
        gb_src_rsrc<DUAL>(nsrc, A, W, more ? M : 0, N, more ? K : 0, ntile.tm, ntile.tn);
        gb_slab<0, true, true>(acc, xa, xb, ya, yb, nsrc, 0, ws, wm, wn, l32, kg);
        gb_slab<1, false, false>(acc, xa, xb, ya, yb, nsrc, 0, ws, wm, wn, l32, kg);
        bare_barrier();  // every wave is done reading stage 1
        gb_issue(gb_s1, nsrc, GB_K, ws);
        gb_epilogue<EPI>(acc, C, Obf, M, N, tile.tm, tile.tn, wm, wn, l32, kg);
        if (!more) break;
        local = nlocal;
        tile = ntile;
        src = nsrc;
    }
}

template <int EPI>
bool launch_big(const u16* A, const u16* W, int M, int N, int K, float* c, u16* out_bf, hipStream_t st) {
    const int nspan = (EPI == EPI_SWIGLU) ? 128 : GB_N;
    if (M < 256 || K % (2 * GB_K) || N % nspan) return false;
    // buffer offsets and ranges are 32-bit: the rows one tile reaches must stay below 2 GiB
    const long long wspan = (EPI == EPI_SWIGLU) ? (long long)N + 128 : GB_N;
    if (wspan * K * 2 >= (1LL << 31) || (long long)GB_M * K * 2 >= (1LL << 31)) return false;
    if ((long long)GB_M * N * 4 >= (1LL << 31)) return false;  // the output rows of one tile
    const int tiles_m = (M + GB_M - 1) / GB_M, tiles_n = N / nspan;
    // grid: a multiple of 8 (workgroups per XCD), at most one workgroup per CU
    const int per_xcd = (tiles_m * tiles_n + 7) / 8;
    const int grid = 8 * std::min(per_xcd, cu_count() / 8);
    hipLaunchKernelGGL((gemm_big_kernel<EPI>), dim3(grid), dim3(256), 0, st, A, W, M, N, K, c, out_bf, tiles_m,
                       tiles_n);
    return true;
}

template <int EPI>
hipError_t launch_gemm(const u16* A, const u16* W, int M, int N, int K, float* c, u16* out_bf,
                       hipStream_t st) {
    if (M <= 16) {
        launch_skinny<EPI, false>(A, nullptr, nullptr, 0.f, W, M, N, K, c, out_bf, st);
    } else if (!launch_big<EPI>(A, W, M, N, K, c, out_bf, st)) {
        const int bn = (EPI == EPI_SWIGLU) ? 64 : BN;
        dim3 grid((N + bn - 1) / bn, (M + BM - 1) / BM);
        hipLaunchKernelGGL((gemm_tiled_kernel<EPI>), grid, dim3(256), 0, st, A, W, M, N, K, c, out_bf);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t gemm_rmsnorm(const float* X, const u16* gain, float eps, const u16* W, int M, int N, int K, int epi,
                        float* c, u16* out_bf, hipStream_t st) {
    switch (epi) {
        case EPI_STORE: launch_skinny<EPI_STORE, true>(nullptr, X, gain, eps, W, M, N, K, c, out_bf, st); break;
        case EPI_ADD: launch_skinny<EPI_ADD, true>(nullptr, X, gain, eps, W, M, N, K, c, out_bf, st); break;
        case EPI_SWIGLU: launch_skinny<EPI_SWIGLU, true>(nullptr, X, gain, eps, W, M, N, K, c, out_bf, st); break;
        default: launch_skinny<EPI_GELU, true>(nullptr, X, gain, eps, W, M, N, K, c, out_bf, st); break;
    }
    return hipGetLastError();
}

bool gemm_fold_supported(int M, int N, int K) { return fold_ok(M, N, K); }

hipError_t gemm_fold_norm(const u16* xg, const float* ps, int nparts, float eps, const u16* Wp, int M, int N, int K,
                          int epi, float* c, u16* out_bf, hipStream_t st, const int32_t* live) {
    if (!fold_ok(M, N, K)) return hipErrorInvalidValue;
    FoldIO io{};
    io.live = live;
    io.ps_in = ps;
    io.nparts = nparts;
    io.eps = eps;
    switch (epi) {
        case EPI_STORE: launch_fold<EPI_STORE, true, false, true>(xg, Wp, M, N, K, c, out_bf, io, st); break;
        case EPI_SWIGLU: launch_fold<EPI_SWIGLU, true, false, true>(xg, Wp, M, N, K, c, out_bf, io, st); break;
        case EPI_GELU: launch_fold<EPI_GELU, true, false, true>(xg, Wp, M, N, K, c, out_bf, io, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t gemm_fold_add(const u16* A, const u16* Wp, int M, int N, int K, float* x, const u16* add_vec,
                         const u16* next_gain, u16* xg_out, float* ps_out, hipStream_t st, const float* add_rows,
                         float* x_save, const int32_t* live) {
    if (!fold_ok(M, N, K)) return hipErrorInvalidValue;
    if ((add_rows || x_save) && !next_gain) return hipErrorInvalidValue;
    FoldIO io{};
    io.live = live;
    io.add_vec = add_vec;
    io.add_rows = add_rows;
    io.x_save = x_save;
    io.next_gain = next_gain;
    io.xg_out = xg_out;
    io.ps_out = ps_out;
    if (next_gain) launch_fold<EPI_ADD, false, true, true>(A, Wp, M, N, K, x, nullptr, io, st);
    else if (add_vec) return hipErrorInvalidValue;
    else launch_fold<EPI_ADD, false, false, true>(A, Wp, M, N, K, x, nullptr, io, st);
    return hipGetLastError();
}

hipError_t pack_weights(const u16* W, long long rows, int K, u16* Wp, hipStream_t st) {
    if (rows % 8 || K % 64) return hipErrorInvalidValue;
    const long long n8 = rows * K / 8;
    const long long blocks = std::min<long long>((n8 + 255) / 256, 16384);
    hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, W, rows, K, Wp);
    return hipGetLastError();
}

hipError_t gemm(const u16* A, const u16* W, int M, int N, int K, int epi, float* c, u16* out_bf,
                hipStream_t st) {
    switch (epi) {
        case EPI_STORE: return launch_gemm<EPI_STORE>(A, W, M, N, K, c, out_bf, st);
        case EPI_ADD: return launch_gemm<EPI_ADD>(A, W, M, N, K, c, out_bf, st);
        case EPI_SWIGLU: return launch_gemm<EPI_SWIGLU>(A, W, M, N, K, c, out_bf, st);
        default: return launch_gemm<EPI_GELU>(A, W, M, N, K, c, out_bf, st);
    }
}

}  // namespace lk
