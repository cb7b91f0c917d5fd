// Attention kernels for gfx950.
//
// The sparse path follows the FlashLoop abstract (arxivdaily.com): attention
// output differences across loops are dominated by a sparse, stable subset of
// key columns, so loops k >= 2 attend over that subset plus a recent window,
// reading a KV that is the previous loop's plus quantized residuals.
//
// * attn_prefill: causal flash attention, v_mfma_f32_32x32x16_bf16.  Scores are
//   formed transposed (S^T = K Q^T) so that every lane owns one query column: the
//   softmax statistics stay per lane (pairs of lanes l, l+32 share a query).  The
//   P^T operand of O^T = V^T P^T comes straight from the score accumulators; the
//   key order inside each 16-key MFMA step is permuted to match the accumulator
//   layout, and V^T is read from the LDS tile with the same permutation.
// * column_mass: the per-column sum of the loop-1 softmax probabilities, keys
//   outer / queries inner, so each column is reduced in one fixed order.
// * attn_rows: one query row (decode token or kept prefill token) over its own
//   column list, split over columns; reconstructs K/V from the store in fp32
//   (base + loop residuals), lanes own keys for q.k and head dims for p.V.
#include "lk_kernels.h"

namespace lk {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// 8 consecutive elements of K or V row (b, g, pos) as bf16 (dequantized if int8).
template <int HD, bool I8>
__device__ __forceinline__ uint4 load_kv8(const KVLayer& kv, int which, int b, int g, int pos, int e0) {
    const long long row = kv_row(kv, b, g, pos);
    if (!I8) return *(const uint4*)((const u16*)kv.base[which] + row * HD + e0);
    const uint2 c = *(const uint2*)((const int8_t*)kv.base[which] + row * HD + e0);
    const float s = h2f(kv.base_scale[which][row * (HD / 32) + e0 / 32]);
    uint32_t w[2] = {c.x, c.y};
    uint4 out;
    uint32_t* o = (uint32_t*)&out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t word = w[q >> 1];
        const int sh = (q & 1) * 16;
        const float a = (float)(int8_t)((word >> sh) & 0xFF) * s;
        const float bb = (float)(int8_t)((word >> (sh + 8)) & 0xFF) * s;
        o[q] = pack_bf2(a, bb);
    }
    return out;
}

// ---------------------------------------------------------------- flash prefill
template <int HD, bool I8>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const u16* __restrict__ Q, KVLayer kv,
                                                           int T, int H, u16* __restrict__ O,
                                                           float* __restrict__ LSE, float sl2) {
    constexpr int KT = 32;
    constexpr int LDV = HD + 8;
    constexpr int CPR = HD / 8;
    constexpr int NCH = 2 * KT * CPR;
    constexpr int PER = (NCH + 255) / 256;
    __shared__ __attribute__((aligned(16))) u16 Ks[2][KT * LDV];
    __shared__ __attribute__((aligned(16))) u16 Vs[2][KT * LDV];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int kg = lane >> 5, l32 = lane & 31;
    const int h = blockIdx.y, b = blockIdx.z;
    const int G = H / kv.Hkv, g = h / G;
    const int qblk = blockIdx.x * 128;
    const int q0 = qblk + w * 32;
    const int qi = q0 + l32;
    const long long ldq = (long long)H * HD;

    bf16x8 qf[HD / 16];
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (qi < T) v = *(const uint4*)(Q + ((long long)b * T + qi) * ldq + h * HD + ks * 16 + kg * 8);
        qf[ks] = as_bf16x8(v);
    }
    f32x16 oacc[HD / 32];
#pragma unroll
    for (int c = 0; c < HD / 32; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[c][i] = 0.f;
    float m_i = -INFINITY, l_i = 0.f;

    const int kend = min(T, qblk + 128);
    const int ntiles = (kend + KT - 1) / KT;
    uint4 regs[PER];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * 256;
            regs[p] = make_uint4(0, 0, 0, 0);
            if (c < NCH) {
                const int which = c / (KT * CPR);
                const int rem = c % (KT * CPR);
                const int key = t * KT + rem / CPR;
                if (key < T) regs[p] = load_kv8<HD, I8>(kv, which, b, g, key, (rem % CPR) * 8);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * 256;
            if (c < NCH) {
                const int which = c / (KT * CPR);
                const int rem = c % (KT * CPR);
                u16* dst = (which ? Vs[buf] : Ks[buf]) + (rem / CPR) * LDV + (rem % CPR) * 8;
                *(uint4*)dst = regs[p];
            }
        }
    };
    load_tile(0);
    store_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        __syncthreads();
        if (t + 1 < ntiles) load_tile(t + 1);
        const int kbase = t * KT;
        if (kbase <= q0 + 31) {
            f32x16 s;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < HD / 16; ++ks) {
                const bf16x8 a = as_bf16x8(*(const uint4*)&Ks[cur][l32 * LDV + ks * 16 + kg * 8]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kbase + 8 * (i >> 2) + 4 * kg + (i & 3);
                const float v = (key <= qi && key < T) ? s[i] * sl2 : -INFINITY;
                s[i] = v;
                mx = fmaxf(mx, v);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_i, mx);
            const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_i - m_new);
            float p[16];
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                p[i] = (s[i] == -INFINITY) ? 0.f : exp2f(s[i] - m_new);
                rs += p[i];
            }
            rs += __shfl_xor(rs, 32);
            l_i = l_i * alpha + rs;
            m_i = m_new;
#pragma unroll
            for (int c = 0; c < HD / 32; ++c)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
            uint4 pu0, pu1;
            pu0.x = pack_bf2(p[0], p[1]);
            pu0.y = pack_bf2(p[2], p[3]);
            pu0.z = pack_bf2(p[4], p[5]);
            pu0.w = pack_bf2(p[6], p[7]);
            pu1.x = pack_bf2(p[8], p[9]);
            pu1.y = pack_bf2(p[10], p[11]);
            pu1.z = pack_bf2(p[12], p[13]);
            pu1.w = pack_bf2(p[14], p[15]);
            const bf16x8 pb0 = as_bf16x8(pu0), pb1 = as_bf16x8(pu1);
#pragma unroll
            for (int c = 0; c < HD / 32; ++c) {
                const int e = c * 32 + l32;
                uint32_t v0[4], v1[4];
#pragma unroll
                for (int jj = 0; jj < 8; jj += 2) {
                    const int ka = (jj < 4) ? 4 * kg + jj : 8 + 4 * kg + (jj - 4);
                    const int kb = ka + 1;
                    v0[jj >> 1] = (uint32_t)Vs[cur][ka * LDV + e] | ((uint32_t)Vs[cur][kb * LDV + e] << 16);
                    v1[jj >> 1] = (uint32_t)Vs[cur][(16 + ka) * LDV + e] |
                                  ((uint32_t)Vs[cur][(16 + kb) * LDV + e] << 16);
                }
                const bf16x8 va0 = as_bf16x8(make_uint4(v0[0], v0[1], v0[2], v0[3]));
                const bf16x8 va1 = as_bf16x8(make_uint4(v1[0], v1[1], v1[2], v1[3]));
                oacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va0, pb0, oacc[c], 0, 0, 0);
                oacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va1, pb1, oacc[c], 0, 0, 0);
            }
        }
        if (t + 1 < ntiles) store_tile(cur ^ 1);
    }
    if (qi < T) {
        const float inv = 1.f / l_i;
        u16* orow = O + ((long long)b * T + qi) * ldq + h * HD;
#pragma unroll
        for (int c = 0; c < HD / 32; ++c)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int e0 = c * 32 + 8 * i4 + 4 * kg;
                uint2 v;
                v.x = pack_bf2(oacc[c][i4 * 4 + 0] * inv, oacc[c][i4 * 4 + 1] * inv);
                v.y = pack_bf2(oacc[c][i4 * 4 + 2] * inv, oacc[c][i4 * 4 + 3] * inv);
                *(uint2*)(orow + e0) = v;
            }
        if (kg == 0) LSE[((long long)b * H + h) * T + qi] = m_i + log2f(l_i);
    }
}

// ---------------------------------------------------------------- column mass
template <int HD, bool I8>
__global__ __launch_bounds__(256) void column_mass_kernel(const u16* __restrict__ Q, KVLayer kv,
                                                          const float* __restrict__ LSE, int T, int H,
                                                          float* __restrict__ mass, float sl2) {
    constexpr int LDQ = HD + 8;
    constexpr int CPR = HD / 8;
    __shared__ __attribute__((aligned(16))) u16 Qs[32 * LDQ];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int kg = lane >> 5, l32 = lane & 31;
    const int g = blockIdx.y, b = blockIdx.z;
    const int Hkv = kv.Hkv, G = H / Hkv;
    const int kblk = blockIdx.x * 128;
    const int j0 = kblk + w * 32;
    const long long ldq = (long long)H * HD;
    bf16x8 kf[HD / 16];
    {
        const int key = j0 + l32;
#pragma unroll
        for (int ks = 0; ks < HD / 16; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (key < T) v = load_kv8<HD, I8>(kv, 0, b, g, key, ks * 16 + kg * 8);
            kf[ks] = as_bf16x8(v);
        }
    }
    float cs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) cs[i] = 0.f;
    const int nqt = (T + 31) / 32;
    for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        for (int qt = kblk / 32; qt < nqt; ++qt) {
            __syncthreads();
            for (int c = tid; c < 32 * CPR; c += 256) {
                const int r = c / CPR, ch = c % CPR;
                const int q = qt * 32 + r;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (q < T) v = *(const uint4*)(Q + ((long long)b * T + q) * ldq + h * HD + ch * 8);
                *(uint4*)&Qs[r * LDQ + ch * 8] = v;
            }
            __syncthreads();
            if (qt * 32 + 31 < j0) continue;
            f32x16 s;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < HD / 16; ++ks) {
                const bf16x8 bq = as_bf16x8(*(const uint4*)&Qs[l32 * LDQ + ks * 16 + kg * 8]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], bq, s, 0, 0, 0);
            }
            const int q = qt * 32 + l32;
            if (q < T) {
                const float lse2 = LSE[((long long)b * H + h) * T + q];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j0 + 8 * (i >> 2) + 4 * kg + (i & 3);
                    if (key <= q) cs[i] += exp2f(s[i] * sl2 - lse2);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float v = cs[i];
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o);
        cs[i] = v;
    }
    if (l32 == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = j0 + 8 * (i >> 2) + 4 * kg + (i & 3);
            if (key < T) mass[((long long)b * Hkv + g) * T + key] = cs[i];
        }
    }
}

// ---------------------------------------------------------------- row attention
// Reconstruct 32 consecutive elements [e0, e0+32) of K/V row (b, g, pos) at loop k.
template <int HD>
__device__ __forceinline__ void recon32(const KVLayer& v, int kv, int b, int g, int pos, int e0, int k,
                                        float* x) {
    const long long row = kv_row(v, b, g, pos);
    if (!v.lazy || v.base_bits == 16) {
        const uint4* src = (const uint4*)((const u16*)v.base[kv] + row * HD + e0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 u = src[q];
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[q * 8 + 2 * j] = __uint_as_float(w4[j] << 16);
                x[q * 8 + 2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
            }
        }
    } else {
        const float s = h2f(v.base_scale[kv][row * (HD / 32) + e0 / 32]);
        const uint4* src = (const uint4*)((const int8_t*)v.base[kv] + row * HD + e0);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint4 u = src[q];
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int t = 0; t < 4; ++t) x[q * 16 + j * 4 + t] = (float)(int8_t)((w4[j] >> (8 * t)) & 0xFF) * s;
        }
    }
    if (!v.lazy) return;
    for (int kk = 2; kk <= k; ++kk) {
        const int sl = v.slot[((long long)(kk - 2) * v.B + b) * v.Tmax + pos];
        if (sl < 0) continue;
        const long long rr = res_row(v, b, g, sl);
        if (v.res_bits == 16) {
            const uint4* src = (const uint4*)((const u16*)v.res[kk - 2][kv] + rr * HD + e0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 u = src[q];
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[q * 8 + 2 * j] = __uint_as_float(w4[j] << 16);
                    x[q * 8 + 2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
                }
            }
        } else {
            const float s = h2f(v.res_scale[kk - 2][kv][rr * (HD / 32) + e0 / 32]);
            if (v.res_bits == 8) {
                const uint4* src = (const uint4*)((const int8_t*)v.res[kk - 2][kv] + rr * HD + e0);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint4 u = src[q];
                    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            x[q * 16 + j * 4 + t] = x[q * 16 + j * 4 + t] +
                                                    (float)(int8_t)((w4[j] >> (8 * t)) & 0xFF) * s;
                }
            } else {
                const uint4 u = *(const uint4*)((const uint8_t*)v.res[kk - 2][kv] + rr * (HD / 2) + e0 / 2);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        int nib = (int)((w4[j] >> (4 * t)) & 0xF);
                        nib = nib >= 8 ? nib - 16 : nib;
                        x[j * 8 + t] = x[j * 8 + t] + (float)nib * s;
                    }
            }
        }
    }
}

template <int HD, int G, bool SPARSE>
__global__ __launch_bounds__(64) void attn_rows_kernel(RowsAttn a) {
    constexpr int DPL = HD >= 64 ? HD / 64 : 1;   // head dims per lane in p.V
    const int row = blockIdx.x, split = blockIdx.y, bg = blockIdx.z;
    const int Hkv = a.kv.Hkv;
    const int b = bg / Hkv, g = bg % Hkv;
    const int lane = threadIdx.x;
    const long long qrow = (long long)b * a.n_rows + row;
    const int pos = a.qpos ? a.qpos[qrow] : a.pos;
    __shared__ float qs[G][HD];
    __shared__ float ps[G][64];
    __shared__ int cs[64];
    const float scale = 1.0f / sqrtf((float)HD);
    for (int idx = lane; idx < G * HD; idx += 64) {
        const int hh = idx / HD, e = idx % HD;
        qs[hh][e] = bf2f(a.q[qrow * a.H * HD + (g * G + hh) * HD + e]) * scale;
    }
    int cntS = 0, win_lo = 0;
    const int32_t* S = nullptr;
    if (SPARSE) {
        S = a.cols + ((long long)b * Hkv + g) * a.n_cols;
        const int lim = pos - a.window;  // S columns at or below lim lie outside the window
        int lo = 0, hi = a.n_cols;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (S[mid] <= lim) lo = mid + 1;
            else hi = mid;
        }
        cntS = lo;
        win_lo = max(0, pos - a.window + 1);
    }
    const int ncols = cntS + (pos - win_lo + 1);
    const int c_begin = split * a.chunk;
    const int c_end = min(ncols, c_begin + a.chunk);
    float m[G], l[G], o[G][DPL];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.f;
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) o[hh][dd] = 0.f;
    }
    __syncthreads();
    for (int c0 = c_begin; c0 < c_end; c0 += 64) {
        const int c = c0 + lane;
        const bool valid = c < c_end;
        const int col = valid ? (c < cntS ? S[c] : win_lo + (c - cntS)) : 0;
        float s[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) s[hh] = 0.f;
        if (valid) {
            for (int e0 = 0; e0 < HD; e0 += 32) {
                float x[32];
                recon32<HD>(a.kv, 0, b, g, col, e0, a.k_loop, x);
#pragma unroll
                for (int hh = 0; hh < G; ++hh)
#pragma unroll
                    for (int e = 0; e < 32; ++e) s[hh] += qs[hh][e0 + e] * x[e];
            }
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float sv = valid ? s[hh] : -INFINITY;
            const float mx = wave_max(sv);
            const float m_new = fmaxf(m[hh], mx);
            const float alpha = (m[hh] == -INFINITY) ? 0.f : expf(m[hh] - m_new);
            const float p = valid ? expf(sv - m_new) : 0.f;
            l[hh] = l[hh] * alpha + wave_sum(p);
            m[hh] = m_new;
#pragma unroll
            for (int dd = 0; dd < DPL; ++dd) o[hh][dd] *= alpha;
            ps[hh][lane] = p;
        }
        cs[lane] = col;
        __syncthreads();
        const int cnt = min(64, c_end - c0);
        const int e = lane * DPL;
        if (e < HD) {
            for (int cc = 0; cc < cnt; ++cc) {
                const int colv = cs[cc];
                float vv[DPL];
#pragma unroll
                for (int dd = 0; dd < DPL; ++dd) vv[dd] = kv_recon_elem(a.kv, 1, b, g, colv, e + dd, a.k_loop);
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    const float pp = ps[hh][cc];
#pragma unroll
                    for (int dd = 0; dd < DPL; ++dd) o[hh][dd] += pp * vv[dd];
                }
            }
        }
        __syncthreads();
    }
    float* P = a.part + ((qrow * Hkv + g) * a.n_splits + split) * (long long)G * (HD + 2);
    const int e = lane * DPL;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        if (e < HD)
#pragma unroll
            for (int dd = 0; dd < DPL; ++dd) P[hh * (HD + 2) + e + dd] = o[hh][dd];
        if (lane == 0) {
            P[hh * (HD + 2) + HD] = m[hh];
            P[hh * (HD + 2) + HD + 1] = l[hh];
        }
    }
}

__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part, int n_splits,
                                                           int G, int HD, int H, int Hkv,
                                                           u16* __restrict__ out) {
    const long long qrow = blockIdx.x;
    const int g = blockIdx.y;
    const float* base = part + (qrow * Hkv + g) * (long long)n_splits * G * (HD + 2);
    for (int idx = threadIdx.x; idx < G * HD; idx += 256) {
        const int hh = idx / HD, e = idx % HD;
        float M = -INFINITY;
        for (int s = 0; s < n_splits; ++s) M = fmaxf(M, base[(long long)s * G * (HD + 2) + hh * (HD + 2) + HD]);
        float L = 0.f, acc = 0.f;
        for (int s = 0; s < n_splits; ++s) {
            const float* ps = base + (long long)s * G * (HD + 2) + hh * (HD + 2);
            const float ms = ps[HD];
            if (ms == -INFINITY) continue;
            const float wgt = expf(ms - M);
            L += wgt * ps[HD + 1];
            acc += wgt * ps[e];
        }
        out[qrow * H * HD + (g * G + hh) * HD + e] = f2bf(acc / L);
    }
}

template <int HD>
hipError_t prefill_hd(const u16* q, const KVLayer& kv, int B, int T, int H, u16* out, float* lse,
                      hipStream_t st) {
    dim3 grid((T + 127) / 128, H, B);
    const float sl2 = kLog2e / sqrtf((float)HD);
    if (kv.lazy && kv.base_bits == 8)
        hipLaunchKernelGGL((attn_prefill_kernel<HD, true>), grid, dim3(256), 0, st, q, kv, T, H, out, lse, sl2);
    else
        hipLaunchKernelGGL((attn_prefill_kernel<HD, false>), grid, dim3(256), 0, st, q, kv, T, H, out, lse, sl2);
    return hipGetLastError();
}

template <int HD>
hipError_t mass_hd(const u16* q, const KVLayer& kv, const float* lse, int B, int T, int H, float* mass,
                   hipStream_t st) {
    dim3 grid((T + 127) / 128, kv.Hkv, B);
    const float sl2 = kLog2e / sqrtf((float)HD);
    if (kv.lazy && kv.base_bits == 8)
        hipLaunchKernelGGL((column_mass_kernel<HD, true>), grid, dim3(256), 0, st, q, kv, lse, T, H, mass, sl2);
    else
        hipLaunchKernelGGL((column_mass_kernel<HD, false>), grid, dim3(256), 0, st, q, kv, lse, T, H, mass, sl2);
    return hipGetLastError();
}

template <int HD, int G>
void rows_launch(const RowsAttn& a, hipStream_t st) {
    dim3 grid(a.n_rows, a.n_splits, a.B * a.kv.Hkv);
    if (a.cols)
        hipLaunchKernelGGL((attn_rows_kernel<HD, G, true>), grid, dim3(64), 0, st, a);
    else
        hipLaunchKernelGGL((attn_rows_kernel<HD, G, false>), grid, dim3(64), 0, st, a);
}

template <int HD>
void rows_hd(const RowsAttn& a, int G, hipStream_t st) {
    switch (G) {
        case 1: rows_launch<HD, 1>(a, st); break;
        case 2: rows_launch<HD, 2>(a, st); break;
        case 4: rows_launch<HD, 4>(a, st); break;
        default: rows_launch<HD, 8>(a, st); break;
    }
}

}  // namespace

hipError_t attn_prefill(const u16* q, const KVLayer& kv, int B, int T, int H, u16* out, float* lse,
                        hipStream_t st) {
    switch (kv.hd) {
        case 32: return prefill_hd<32>(q, kv, B, T, H, out, lse, st);
        case 64: return prefill_hd<64>(q, kv, B, T, H, out, lse, st);
        default: return prefill_hd<128>(q, kv, B, T, H, out, lse, st);
    }
}

hipError_t column_mass(const u16* q, const KVLayer& kv, const float* lse, int B, int T, int H,
                       float* mass, hipStream_t st) {
    switch (kv.hd) {
        case 32: return mass_hd<32>(q, kv, lse, B, T, H, mass, st);
        case 64: return mass_hd<64>(q, kv, lse, B, T, H, mass, st);
        default: return mass_hd<128>(q, kv, lse, B, T, H, mass, st);
    }
}

hipError_t attn_rows_main(const RowsAttn& a, hipStream_t st) {
    const int G = a.H / a.kv.Hkv;
    switch (a.kv.hd) {
        case 32: rows_hd<32>(a, G, st); break;
        case 64: rows_hd<64>(a, G, st); break;
        default: rows_hd<128>(a, G, st); break;
    }
    return hipGetLastError();
}

hipError_t attn_rows_combine(const RowsAttn& a, hipStream_t st) {
    const int G = a.H / a.kv.Hkv;
    dim3 grid(a.B * a.n_rows, a.kv.Hkv);
    hipLaunchKernelGGL(attn_combine_kernel, grid, dim3(256), 0, st, a.part, a.n_splits, G, a.kv.hd, a.H,
                       a.kv.Hkv, a.out);
    return hipGetLastError();
}

}  // namespace lk
