// Elementwise, selection and KV-store-write kernels for gfx950.
//
// Token-sparse update and residual quantization follow the FlashLoop abstract
// (arxivdaily.com, "FlashLoop: Fast and Memory-Efficient Looped Transformers
// via Lazy Updates"); the loop embedding and RoPE follow the FlashLoop
// walk-through (discosf.com, section 3.2).
#include "lk_kernels.h"

namespace lk {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void embed_kernel(const int32_t* ids, const u16* tok, float* h,
                                                         int d, int vocab) {
    const int r = blockIdx.x;
    const int id = min(max(ids[r], 0), vocab - 1);  // out-of-range ids read row 0 / vocab-1
    const long long src = (long long)id * d;
    float* dst = h + (long long)r * d;
    for (int j = threadIdx.x; j < d; j += kThreads) dst[j] = bf2f(tok[src + j]);
}

// x += add (optional); xg = x * gain as lane-packed float16; ps[r] = sum of x^2 over the
// row.
__global__ __launch_bounds__(kThreads) void norm_prep_kernel(float* x, const u16* add, const u16* gain, int d,
                                                             u16* xg, float* ps) {
    __shared__ float red[16];
    const int r = blockIdx.x;
    float* row = x + (long long)r * d;
    float ss = 0.f;
    for (int j = threadIdx.x; j < d; j += kThreads) {
        float v = row[j];
        if (add) {
            v = v + bf2f(add[j]);
            row[j] = v;
        }
        const long long pi = pk_index(r, j, d);
        xg[pi] = f2h_bits(v * bf2f(gain[j]));
        ss += v * v;
    }
    ss = block_sum(ss, red);
    if (threadIdx.x == 0) ps[r] = ss;
}

__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(float* x, const u16* add, const u16* gain,
                                                           float eps, int d, u16* out_bf,
                                                           float* out_f32) {
    __shared__ float red[16];
    const int r = blockIdx.x;
    float* row = x + (long long)r * d;
    float ss = 0.f;
    constexpr int MV = 4;  // float4 per thread held in registers (d <= 4096)
    if (d % (4 * kThreads) == 0 && d <= MV * 4 * kThreads) {
        const int nv = d / (4 * kThreads);
        float4 v[MV];
#pragma unroll
        for (int k = 0; k < MV; ++k) {
            if (k >= nv) break;
            const int j = (k * kThreads + threadIdx.x) * 4;
            float4 a = *(const float4*)(row + j);
            if (add) {
                const uint2 ad = *(const uint2*)(add + j);
                a.x = a.x + __uint_as_float(ad.x << 16);
                a.y = a.y + __uint_as_float(ad.x & 0xFFFF0000u);
                a.z = a.z + __uint_as_float(ad.y << 16);
                a.w = a.w + __uint_as_float(ad.y & 0xFFFF0000u);
                *(float4*)(row + j) = a;
            }
            v[k] = a;
            ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
        }
        ss = block_sum(ss, red);
        const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
        for (int k = 0; k < MV; ++k) {
            if (k >= nv) break;
            const int j = (k * kThreads + threadIdx.x) * 4;
            const uint2 gv = *(const uint2*)(gain + j);
            const float y0 = (v[k].x * inv) * __uint_as_float(gv.x << 16);
            const float y1 = (v[k].y * inv) * __uint_as_float(gv.x & 0xFFFF0000u);
            const float y2 = (v[k].z * inv) * __uint_as_float(gv.y << 16);
            const float y3 = (v[k].w * inv) * __uint_as_float(gv.y & 0xFFFF0000u);
            if (out_bf) *(uint2*)(out_bf + (long long)r * d + j) = make_uint2(pack_bf2(y0, y1), pack_bf2(y2, y3));
            else *(float4*)(out_f32 + (long long)r * d + j) = make_float4(y0, y1, y2, y3);
        }
        return;
    }
    for (int j = threadIdx.x; j < d; j += kThreads) {
        float v = row[j];
        if (add) {
            v = v + bf2f(add[j]);
            row[j] = v;
        }
        ss += v * v;
    }
    ss = block_sum(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
    for (int j = threadIdx.x; j < d; j += kThreads) {
        const float y = (row[j] * inv) * bf2f(gain[j]);
        if (out_bf) out_bf[(long long)r * d + j] = f2bf(y);
        else out_f32[(long long)r * d + j] = y;
    }
}

__global__ __launch_bounds__(kThreads) void add_rows_kernel(float* x, const u16* add, int d) {
    float* row = x + (long long)blockIdx.x * d;
    for (int j = threadIdx.x; j < d; j += kThreads) row[j] = row[j] + bf2f(add[j]);
}

__global__ void add_f32_kernel(float* x, const float* y, long long n) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        x[i] = x[i] + y[i];
}

__global__ void copy_f32_kernel(const float* s, float* d, long long n) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        d[i] = s[i];
}
// Decode-time loop skipping, at the start of a loop k >= 2: row b (one block) still in
// the loops computes key = sum_e (src - prev)^2, its state change over loop k-1, leaves
// the loops when key < tau, and sets prev = src (h_{k-1}: the next loop's h_{k-2}, and
// the final state of a row that left).  Rows already out are not touched.
__global__ __launch_bounds__(256) void skip_gate_kernel(const float* __restrict__ src, float* __restrict__ prev,
                                                        int32_t* __restrict__ act, int32_t* __restrict__ live,
                                                        float tau, int d) {
    __shared__ float red[16];
    const int b = blockIdx.x;
    if (!act[b]) return;
    const float* x = src + (long long)b * d;
    float* y = prev + (long long)b * d;
    float v = 0.f;
    for (int e = threadIdx.x; e < d; e += blockDim.x) {
        const float t = x[e] - y[e];
        v += t * t;
    }
    const float key = block_sum(v, red);
    for (int e = threadIdx.x; e < d; e += blockDim.x) y[e] = x[e];
    if (threadIdx.x == 0 && key < tau) {
        act[b] = 0;
        atomicSub(live, 1);
    }
}
// After the last loop: rows that left take back their final state.
__global__ void skip_restore_kernel(float* __restrict__ h, const float* __restrict__ prev,
                                    const int32_t* __restrict__ act, int d) {
    const int b = blockIdx.x;
    if (act[b]) return;
    for (int e = threadIdx.x; e < d; e += blockDim.x) h[(long long)b * d + e] = prev[(long long)b * d + e];
}
__global__ void fill_i32_kernel(int32_t* p, int32_t v, long long n) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        p[i] = v;
}
__global__ void add_i32_kernel(int32_t* p, int32_t v) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p += v;
}
__global__ void fill_f32_kernel(float* p, float v, long long n) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ __launch_bounds__(kThreads) void delta_kernel(const float* a, const float* b, int d,
                                                         float* key) {
    __shared__ float red[16];
    const long long off = (long long)blockIdx.x * d;
    float s = 0.f;
    for (int j = threadIdx.x; j < d; j += kThreads) {
        const float t = a[off + j] - b[off + j];
        s += t * t;
    }
    s = block_sum(s, red);
    if (threadIdx.x == 0) key[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void gather_kernel(const float* h, const int32_t* idx, int n,
                                                          int T, int d, const u16* add, float* xc,
                                                          int32_t* slot_map, int Tmax, const float* add_src) {
    const int r = blockIdx.x;  // compact row b*n + j
    const int b = r / n, j = r % n;
    const int i = idx[r];
    const float* src = h + ((long long)b * T + i) * d;
    const float* src2 = add_src ? add_src + ((long long)b * T + i) * d : nullptr;
    float* dst = xc + (long long)r * d;
    for (int c = threadIdx.x; c < d; c += kThreads) {
        float v = src[c];
        if (src2) v = v + src2[c];
        dst[c] = v + (add ? bf2f(add[c]) : 0.f);
    }
    if (slot_map && threadIdx.x == 0) slot_map[(long long)b * Tmax + i] = j;
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(const float* xc, const int32_t* idx, int n,
                                                           int T, int d, float* h, float* key) {
    __shared__ float red[16];
    const int r = blockIdx.x;
    const int b = r / n;
    const int i = idx[r];
    float* dst = h + ((long long)b * T + i) * d;
    const float* src = xc + (long long)r * d;
    float s = 0.f;
    for (int c = threadIdx.x; c < d; c += kThreads) {
        const float t = src[c] - dst[c];
        s += t * t;
    }
    if (key) {
        s = block_sum(s, red);
        if (threadIdx.x == 0) key[(long long)b * T + i] = s;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < d; c += kThreads) dst[c] = src[c];
}

// ---------------------------------------------------------------- top-n selector
// Order-preserving map of a finite float to uint32 (larger float -> larger key);
// -0 is mapped like +0 so that equal floats give equal keys.
__device__ __forceinline__ uint32_t ord_key(float f) {
    if (f == 0.f) f = 0.f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive block scan of one int per thread (256 threads); *total = block sum.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) sh[w] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
        if (i < w) off += sh[i];
        tot += sh[i];
    }
    *total = tot;
    return off + x - v;
}

// Radix select of the n-th largest key, then an index-ordered compaction that keeps
// every key above it and the lowest-index ties: the result equals a stable sort by
// (key descending, index ascending) cut at n, listed in ascending index order.
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* keys, int cols, int n, int32_t* out) {
    __shared__ int hist[256];
    __shared__ int sh[8];
    __shared__ uint32_t s_prefix;
    __shared__ int s_need;
    const int row = blockIdx.x;
    const float* k = keys + (long long)row * cols;
    int32_t* o = out + (long long)row * n;
    uint32_t prefix = 0, mask = 0;
    int need = n;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += kThreads) hist[i] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < cols; i += kThreads) {
            const uint32_t u = ord_key(k[i]);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int cum = 0, dsel = 0;
            for (int dg = 255; dg >= 0; --dg) {
                if (cum + hist[dg] >= need) {
                    dsel = dg;
                    break;
                }
                cum += hist[dg];
            }
            s_prefix = prefix | ((uint32_t)dsel << shift);
            s_need = need - cum;
        }
        __syncthreads();
        prefix = s_prefix;
        need = s_need;
        mask |= 255u << shift;
        __syncthreads();
    }
    const uint32_t tau = prefix;  // n-th largest key; `need` ties of it are kept
    int taken = 0, eq_seen = 0;
    for (int c0 = 0; c0 < cols; c0 += kThreads) {
        const int i = c0 + threadIdx.x;
        uint32_t u = 0;
        if (i < cols) u = ord_key(k[i]);
        const int gt = (i < cols) && (u > tau);
        const int eq = (i < cols) && (u == tau);
        int eq_tot, take_tot;
        const int eq_rank = block_excl_scan(eq, sh, &eq_tot) + eq_seen;
        const int take = gt || (eq && eq_rank < need);
        const int p = block_excl_scan(take, sh + 4, &take_tot) + taken;
        if (take && p < n) o[p] = i;
        taken += take_tot;
        eq_seen += eq_tot;
    }
}

// ---------------------------------------------------------------- quantizer (test entry)
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(const float* x, long long groups,
                                                                 int hd, int bits, uint8_t* codes,
                                                                 u16* scales) {
    const long long gi = (long long)blockIdx.x * (kThreads / 32) + (threadIdx.x >> 5);
    if (gi >= groups) return;  // whole 32-lane groups leave together
    const int lane = threadIdx.x & 31;
    const int gpr = hd / 32;
    const long long row = gi / gpr;
    const int e = (int)(gi % gpr) * 32 + lane;
    const float r = x[row * hd + e];
    u16 sb;
    const int qmax = (1 << (bits - 1)) - 1;
    const int c = quant_group32(r, qmax, &sb);
    if (lane == 0) scales[gi] = sb;
    if (bits == 8) {
        codes[row * hd + e] = (uint8_t)(int8_t)c;
    } else {
        const int other = __shfl_xor(c, 1);
        if ((lane & 1) == 0)
            codes[row * (hd / 2) + e / 2] = (uint8_t)((c & 0xF) | ((other & 0xF) << 4));
    }
}

// ---------------------------------------------------------------- RoPE + KV write
}  // namespace

// RoPE angles: inv_freq (float64) is passed by value.
struct InvFreq {
    double v[64];
};

namespace {

// Block (row r, unit u), 128 threads.  Units [0, nq) rotate q heads (256/hd heads per
// unit, one (head, pair index) per thread); unit nq + kv*Hkv + g handles K (kv = 0,
// rotated) or V (kv = 1) head g: thread e owns element e and writes it to the store
// (32-lane groups quantize together).
__global__ __launch_bounds__(128) void rope_kv_write_kernel(const float* qkv, int rows_per_seq,
                                                            const int32_t* pos_arr, int pos_offset,
                                                            int H, int Hkv, int hd, InvFreq inv,
                                                            u16* q_out, int q_half, KVWrite w) {
    const int r = blockIdx.x, u = blockIdx.y, t = threadIdx.x;
    const int b = r / rows_per_seq;
    const int iseq = r % rows_per_seq;
    const int t0 = w.dpos ? *w.dpos : pos_offset;
    const int pos = pos_arr ? pos_arr[r] : t0 + iseq;
    const int half = hd / 2;
    const float* src = qkv + (long long)r * (H + 2 * Hkv) * hd;
    const int qpb = 256 / hd;
    const int nq = (H + qpb - 1) / qpb;
    const bool tab = w.rope_tab && pos < w.rope_rows;
    if (u < nq) {
        const int hh = u * qpb + t / half, i = t % half;
        if (hh >= H) return;
        float c, sn;
        if (w.rope_cs) {
            c = w.rope_cs[2 * i];
            sn = w.rope_cs[2 * i + 1];
        } else if (tab) {
            c = w.rope_tab[((long long)pos * half + i) * 2];
            sn = w.rope_tab[((long long)pos * half + i) * 2 + 1];
        } else {
            double sd, cd;
            sincos((double)pos * inv.v[i], &sd, &cd);
            c = (float)cd;
            sn = (float)sd;
        }
        const float x1 = src[hh * hd + i], x2 = src[hh * hd + i + half];
        u16* dq = q_out + (long long)r * H * hd + hh * hd;
        const float r1 = rope_lo(x1, x2, c, sn), r2 = rope_hi(x1, x2, c, sn);
        if (w.range_flag && !(fabsf(r1) <= 65504.f && fabsf(r2) <= 65504.f)) *w.range_flag = 1u;
        dq[i] = q_half ? f2h_bits(r1) : f2bf(r1);
        dq[i + half] = q_half ? f2h_bits(r2) : f2bf(r2);
        return;
    }
    const int kv = (u - nq) / Hkv, g = (u - nq) % Hkv;
    const int e = t;
    if (e >= hd) return;  // whole 32-lane groups (hd is a multiple of 32)
    float c = 1.f, sn = 0.f;
    if (kv == 0) {
        const int i = e % half;
        if (w.rope_cs) {
            c = w.rope_cs[2 * i];
            sn = w.rope_cs[2 * i + 1];
        } else if (tab) {
            c = w.rope_tab[((long long)pos * half + i) * 2];
            sn = w.rope_tab[((long long)pos * half + i) * 2 + 1];
        } else {
            double sd, cd;
            sincos((double)pos * inv.v[i], &sd, &cd);
            c = (float)cd;
            sn = (float)sd;
        }
    }
    kv_write_elem(src, H, Hkv, hd, b, g, kv, e, pos, iseq, c, sn, w, u == nq && t == 0);
}

inline int grid_for(long long n) {
    long long g = (n + kThreads - 1) / kThreads;
    return (int)(g > 65536 ? 65536 : (g < 1 ? 1 : g));
}

}  // namespace

hipError_t embed(const int32_t* ids, const u16* tok_emb, float* h, int rows, int d, int vocab,
                 hipStream_t st) {
    hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(kThreads), 0, st, ids, tok_emb, h, d, vocab);
    return hipGetLastError();
}

hipError_t rmsnorm(float* x, const u16* add, const u16* gain, float eps, int rows, int d, u16* out_bf,
                   float* out_f32, hipStream_t st) {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(kThreads), 0, st, x, add, gain, eps, d, out_bf,
                       out_f32);
    return hipGetLastError();
}

hipError_t norm_prep(float* x, const u16* add, const u16* gain, int rows, int d, u16* xg, float* ps,
                     hipStream_t st) {
    if (rows > 8 || d % 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL(norm_prep_kernel, dim3(rows), dim3(kThreads), 0, st, x, add, gain, d, xg, ps);
    return hipGetLastError();
}

hipError_t add_rows(float* x, const u16* add, int rows, int d, hipStream_t st) {
    hipLaunchKernelGGL(add_rows_kernel, dim3(rows), dim3(kThreads), 0, st, x, add, d);
    return hipGetLastError();
}

hipError_t add_f32(float* x, const float* y, long long n, hipStream_t st) {
    hipLaunchKernelGGL(add_f32_kernel, dim3(grid_for(n)), dim3(kThreads), 0, st, x, y, n);
    return hipGetLastError();
}
hipError_t copy_f32(const float* src, float* dst, long long n, hipStream_t st) {
    hipLaunchKernelGGL(copy_f32_kernel, dim3(grid_for(n)), dim3(kThreads), 0, st, src, dst, n);
    return hipGetLastError();
}
hipError_t skip_gate(const float* src, float* prev, int32_t* act, int32_t* live, float tau, int B, int d,
                     hipStream_t st) {
    hipLaunchKernelGGL(skip_gate_kernel, dim3(B), dim3(256), 0, st, src, prev, act, live, tau, d);
    return hipGetLastError();
}
hipError_t skip_restore(float* h, const float* prev, const int32_t* act, int B, int d, hipStream_t st) {
    hipLaunchKernelGGL(skip_restore_kernel, dim3(B), dim3(256), 0, st, h, prev, act, d);
    return hipGetLastError();
}
hipError_t fill_i32(int32_t* p, int32_t v, long long n, hipStream_t st) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(n)), dim3(kThreads), 0, st, p, v, n);
    return hipGetLastError();
}
hipError_t add_i32(int32_t* p, int32_t v, hipStream_t st) {
    hipLaunchKernelGGL(add_i32_kernel, dim3(1), dim3(64), 0, st, p, v);
    return hipGetLastError();
}
__global__ void iota_rows_kernel(int32_t* p, int n, long long total) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total; i += (long long)gridDim.x * blockDim.x)
        p[i] = (int32_t)(i % n);
}
hipError_t iota_rows(int32_t* p, int rows, int n, hipStream_t st) {
    const long long total = (long long)rows * n;
    hipLaunchKernelGGL(iota_rows_kernel, dim3(grid_for(total)), dim3(kThreads), 0, st, p, n, total);
    return hipGetLastError();
}
hipError_t fill_f32(float* p, float v, long long n, hipStream_t st) {
    hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(kThreads), 0, st, p, v, n);
    return hipGetLastError();
}

hipError_t delta_keys(const float* a, const float* b, int rows, int d, float* key, hipStream_t st) {
    hipLaunchKernelGGL(delta_kernel, dim3(rows), dim3(kThreads), 0, st, a, b, d, key);
    return hipGetLastError();
}

hipError_t gather_rows(const float* h, const int32_t* idx, int B, int n, int T, int d, const u16* add,
                       float* xc, int32_t* slot_map, int Tmax, hipStream_t st, const float* add_src) {
    hipLaunchKernelGGL(gather_kernel, dim3(B * n), dim3(kThreads), 0, st, h, idx, n, T, d, add, xc,
                       slot_map, Tmax, add_src);
    return hipGetLastError();
}

hipError_t scatter_rows(const float* xc, const int32_t* idx, int B, int n, int T, int d, float* h,
                        float* key, hipStream_t st) {
    hipLaunchKernelGGL(scatter_kernel, dim3(B * n), dim3(kThreads), 0, st, xc, idx, n, T, d, h, key);
    return hipGetLastError();
}

hipError_t topk_rows(const float* keys, int rows, int cols, int n, int32_t* out, hipStream_t st) {
    hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(kThreads), 0, st, keys, cols, n, out);
    return hipGetLastError();
}

hipError_t quantize_rows(const float* x, int rows, int hd, int bits, uint8_t* codes, u16* scales,
                         hipStream_t st) {
    const long long groups = (long long)rows * (hd / 32);
    const int per_block = kThreads / 32;
    const long long blocks = (groups + per_block - 1) / per_block;
    hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, x, groups,
                       hd, bits, codes, scales);
    return hipGetLastError();
}

__global__ void rope_angles_kernel(const int32_t* dpos, InvFreq inv, int half, float* cs) {
    const int i = threadIdx.x;
    if (i >= half) return;
    double sd, cd;
    sincos((double)*dpos * inv.v[i], &sd, &cd);
    cs[2 * i] = (float)cd;
    cs[2 * i + 1] = (float)sd;
}

hipError_t rope_angles(const int32_t* dpos, const double* inv_freq, int hd, float* cs, hipStream_t st) {
    InvFreq inv;
    for (int i = 0; i < hd / 2; ++i) inv.v[i] = inv_freq[i];
    hipLaunchKernelGGL(rope_angles_kernel, dim3(1), dim3(64), 0, st, dpos, inv, hd / 2, cs);
    return hipGetLastError();
}

__global__ void rope_table_kernel(InvFreq inv, int T, int half, float* tab) {
    const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
    if (i >= (long long)T * half) return;
    const int p = (int)(i / half), k = (int)(i % half);
    double sd, cd;
    sincos((double)p * inv.v[k], &sd, &cd);
    tab[2 * i] = (float)cd;
    tab[2 * i + 1] = (float)sd;
}

hipError_t rope_table(const double* inv_freq, int T, int hd, float* tab, hipStream_t st) {
    InvFreq inv;
    for (int i = 0; i < hd / 2; ++i) inv.v[i] = inv_freq[i];
    const long long n = (long long)T * (hd / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, inv, T, hd / 2, tab);
    return hipGetLastError();
}

hipError_t rope_kv_write(const float* qkv, int rows, int rows_per_seq, const int32_t* pos, int pos_offset,
                         int H, int Hkv, int hd, const double* inv_freq, u16* q_out, const KVWrite& kvw,
                         hipStream_t st, int q_half) {
    InvFreq inv;
    for (int i = 0; i < hd / 2; ++i) inv.v[i] = inv_freq[i];
    const int qpb = 256 / hd;
    const int units = (H + qpb - 1) / qpb + 2 * Hkv;
    hipLaunchKernelGGL(rope_kv_write_kernel, dim3(rows, units), dim3(128), 0, st, qkv, rows_per_seq, pos,
                       pos_offset, H, Hkv, hd, inv, q_out, q_half, kvw);
    return hipGetLastError();
}

}  // namespace lk
